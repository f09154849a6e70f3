// launch.hpp -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace cas {

enum ElemCode { E_F32 = 0, E_BF16 = 1, E_F16 = 2 };

struct GemmArgs {
    const void *X;
    const void *W;
    float *Y;
    int64_t M, N, K, ldx, ldw, ldy;
    bool predicated = false; // bounds checks inside the MFMA loop (local-padding A/B)
    int64_t batch = 1;       // independent products; batch b reads X + b*bsx, W + b*bsw, writes Y + b*bsy
    int64_t bsx = 0, bsw = 0, bsy = 0; // batch strides in elements
};

struct TrimulArgs {
    const void *qkv;
    void *out;
    int64_t B, T, C, NH, HS;
    float scale;
    bool vec_store; // output rows 16-byte aligned: T * out_bytes % 16 == 0 and out 16-byte aligned
    int out_kind;   // 0 fp32, 1 bfloat16, 2 binary16 (the cas_dtype codes)
    const float *row_max = nullptr;    // causal softmax: per-row statistics (B, NH, T)
    const float *row_logsum = nullptr;
};

// Persistent grids: workgroups of one kernel resident on a device at once
// (occupancy per compute unit times compute units), found once per device.
// Each launcher keeps one ResidentSlots per kernel instance as a static; the
// per-device once_flag makes the first fill safe under concurrent host threads.
struct ResidentSlots {
    static constexpr int MAX_DEV = 64;
    std::once_flag once[MAX_DEV];
    int64_t slots[MAX_DEV] = {};
};

template <class F> int64_t resident_slots(ResidentSlots &c, F kern, int threads)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= ResidentSlots::MAX_DEV) dev = 0;
    std::call_once(c.once[dev], [&c, kern, threads, dev] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, 0) != hipSuccess || n < 1) n = 1;
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 1) cu = 256;
        c.slots[dev] = (int64_t)n * cu;
    });
    return c.slots[dev];
}

// Tile shapes the dense launcher can pick (exposed for tests and tuning).
enum GemmTile { GEMM_TILE_AUTO = 0, GEMM_TILE_64 = 1, GEMM_TILE_128 = 2, GEMM_TILE_256 = 3 };

// vec: elements per global load (a power of two that divides K, both pitches
// and both base addresses' alignment in elements). Returns the launch error.
hipError_t launch_gemm_nt(const GemmArgs &a, int elem, int vec, int tile, hipStream_t s);
int64_t gemm_nt_workgroups(const GemmArgs &a, int elem, int tile);

// 256 x 256 tiles with loads straight into LDS (gemm_nt_wide.hip): 16-bit
// inputs whose rows split into 16-byte pieces (vec * es == 16).
bool gemm_wide_fits(const GemmArgs &a, int es, int vec);
int64_t gemm_wide_workgroups(const GemmArgs &a);
hipError_t launch_gemm_wide(const GemmArgs &a, int elem, hipStream_t s);
// The same kernel for 16-bit rows not in 16-byte pieces (elements at their
// alignment, K >= 8): the first K - K % 8 columns, then a tail kernel adding
// the last K % 8 into Y.
bool gemm_wide_fits_unaligned(const GemmArgs &a, int es);
hipError_t launch_gemm_wide_unaligned(const GemmArgs &a, int elem, hipStream_t s);
// Y += X[:, K0:K] W[:, K0:K]^T for the last K - K0 < 8 columns (batch 1).
bool gemm_ktail_fits(const GemmArgs &a);
hipError_t launch_gemm_ktail(const GemmArgs &a, int elem, int64_t K0, hipStream_t s);

// 64 x 64 fp32 tiles with loads straight into LDS (gemm_nt_direct.hip): rows
// and bases 8-byte aligned (vec >= 2), not predicated.
bool gemm_direct_fits(const GemmArgs &a, int elem, int vec);
hipError_t launch_gemm_direct(const GemmArgs &a, hipStream_t s);

hipError_t launch_trimul(const TrimulArgs &a, int elem, int vec, hipStream_t s);
int64_t trimul_workgroups(int64_t B, int64_t T, int64_t NH);

// Causal softmax (softmax.hip): row statistics into a.row_max / a.row_logsum,
// then the softmax rows (mode 0 log-probabilities, 1 probabilities) into
// a.out. Both need softmax_fits() (heads of up to 512 bytes in 16-byte
// pieces); vec as for launch_trimul.
bool softmax_fits(int64_t T, int64_t HS, int es, int vec);
int64_t row_stats_workgroups(int64_t B, int64_t T, int64_t NH);
hipError_t launch_row_stats(const TrimulArgs &a, int elem, hipStream_t s);
hipError_t launch_softmax(const TrimulArgs &a, int elem, int mode, hipStream_t s);
// Both in one launch: statistics written through a.row_max / a.row_logsum.
hipError_t launch_softmax_fused(const TrimulArgs &a, int elem, int mode, hipStream_t s);
// Attention output (B, T, C) fp32 into a.out from a.row_max / a.row_logsum,
// by input type (softmax_{f32,bf16,f16}.hip).
hipError_t launch_attention_f32(const TrimulArgs &a, hipStream_t s);
hipError_t launch_attention_bf16(const TrimulArgs &a, hipStream_t s);
hipError_t launch_attention_f16(const TrimulArgs &a, hipStream_t s);
// Single pass: y into a.out (16-byte stores when a.vec_store) and the row
// statistics written through a.row_max / a.row_logsum.
hipError_t launch_attention_online_f32(const TrimulArgs &a, hipStream_t s);
hipError_t launch_attention_online_bf16(const TrimulArgs &a, hipStream_t s);
hipError_t launch_attention_online_f16(const TrimulArgs &a, hipStream_t s);
// 16-bit heads of 257 .. 512 bytes (softmax_wide16.hip), elem E_BF16 or E_F16.
hipError_t launch_row_stats_wide16(const TrimulArgs &a, int elem, hipStream_t s);
hipError_t launch_attention_wide16(const TrimulArgs &a, int elem, hipStream_t s);
hipError_t launch_attention_online_wide16(const TrimulArgs &a, int elem, hipStream_t s);

// General shapes (softmax_general.hip): heads whose rows do not split into
// 16-byte pieces or exceed 512 bytes, any head size, within
// general_softmax_fits(). The same outputs as above: row statistics; softmax
// rows (a.out_kind picks the output type); the attention output, with the
// statistics computed and written first when with_stats, else read.
bool general_softmax_fits(int64_t B, int64_t T, int64_t NH, int es, const void *qkv);
hipError_t launch_gen_row_stats(const TrimulArgs &a, int elem, hipStream_t s);
hipError_t launch_gen_softmax(const TrimulArgs &a, int elem, int mode, hipStream_t s);
hipError_t launch_gen_attention(const TrimulArgs &a, int elem, bool with_stats, hipStream_t s);

} // namespace cas
