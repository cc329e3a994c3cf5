// device.hpp -- gfx950 device helpers shared by the dispatch/combine kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kFp8Block = 128;   // channels per FP8 scale, per token

// ---- bfloat16 ------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Two fp32 values -> two bf16 (round to nearest even), `lo` in bits 0..15: one
// v_cvt_pk_bf16_f32 on gfx950.  Converted one by one, each value took its own
// conversion and the pair a shift and an OR to pack.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 8 bf16 in a 16-byte vector -> 8 fp32
__device__ __forceinline__ void unpack8_bf16(const uint4& v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint4 pack8_bf16(const float (&f)[8]) {
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]);
    v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]);
    v.w = pack_bf16x2(f[6], f[7]);
    return v;
}

// ---- 16-byte global accesses with a cache policy ----------------------------------
// Streaming (NT = true) marks loads and stores nontemporal, for buffers far larger
// than the last-level cache; measured on gfx950 it lifts large permuted copies
// from ~5.2 to ~6.1 TB/s but slows copies whose data is still cache resident.

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4* p) {
    if constexpr (NT) {
        const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        return make_uint4(t.x, t.y, t.z, t.w);
    } else {
        return *p;
    }
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ uint2 ld8(const uint2* p) {
    if constexpr (NT) {
        const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        return make_uint2(t.x, t.y);
    } else {
        return *p;
    }
}

template <bool NT>
__device__ __forceinline__ void st16(uint4* p, const uint4& v) {
    if constexpr (NT) {
        const u32x4_t t = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
    } else {
        *p = v;
    }
}

// Store of 16 bytes at unit u of row `row` (of `units` 16-byte units) of a
// buffer, for kernels in which every active lane of the wave stores into the
// same row (each lane its own unit).  Streaming (NT = true): a nontemporal
// global store.  Otherwise a buffer store with the device-scope cache policy
// (SC1): the line is written through the XCD's L2 to the device's coherence
// point while the kernel runs, so no dirty lines are left for the write-back
// at the kernel boundary, and the next kernel, whose workgroups read the row
// from any XCD, finds it there.  Measured on gfx950 against write-back stores,
// per step of the whole path: 128 tokens x top-8 x 7168, 32.3 -> 30.4 us;
// 2048 tokens x top-2 FP8, 72.2 -> 68.6 us; and the pack of 8192 tokens x
// top-8, 93.8 -> 89.8 us.  The buffer's record count is the row's bytes, so
// the hardware drops any store past the row.
constexpr int kRawBufferWord3 = 0x00020000;   // word 3 of a raw (untyped) gfx9 buffer resource
constexpr int kStoreDeviceScope = 16;         // cache-policy operand: SC1

template <bool NT>
__device__ __forceinline__ void st16_row(uint4* base, int row, int units, int u, const uint4& v) {
    if constexpr (NT) {
        st16<true>(&base[(size_t)row * units + u], v);
    } else {
        const int r = __builtin_amdgcn_readfirstlane(row);   // the same in every active lane
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(base + (size_t)r * units, (short)0, units * 16, kRawBufferWord3);
        const u32x4_t t = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(t, rsrc, u * 16, 0, kStoreDeviceScope);
    }
}

// Write-through store (the device-scope cache policy, SC1, as st16_row) of
// element i of row `row` of an array of rows of `count` 4- or 16-byte elements,
// for the small per-row arrays (FP8 scales, handle records) that a kernel writes
// beside its write-through rows and the next kernel reads from other XCDs.  The
// row must be the same in every active lane; the buffer's record count is the
// row's bytes, so the hardware drops any store past the row.
template <typename T>
__device__ __forceinline__ void st_through_row(T* base, int row, int count, int i, const T& v) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 16, "4- or 16-byte elements");
    const int r = __builtin_amdgcn_readfirstlane(row);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(base + (size_t)r * count, (short)0,
                                                                          count * (int)sizeof(T), kRawBufferWord3);
    if constexpr (sizeof(T) == 4) {
        uint32_t w;
        __builtin_memcpy(&w, &v, 4);
        __builtin_amdgcn_raw_buffer_store_b32(w, rsrc, i * 4, 0, kStoreDeviceScope);
    } else {
        u32x4_t w;
        __builtin_memcpy(&w, &v, 16);
        __builtin_amdgcn_raw_buffer_store_b128(w, rsrc, i * 16, 0, kStoreDeviceScope);
    }
}

// ---- OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 significand bits,
// largest finite 448, NaN = S.1111.111, no infinities) ------------------------------
// gfx950's v_cvt_pk_fp8_f32 / v_cvt_pk_f32_fp8 work in this format with round
// to nearest even.  Tested bit for bit against the format's definition on the
// GPU: the encoder on every bf16 value of magnitude <= 448 (ties, subnormals and
// signed zeros included) and on the quotients of the FP8 workloads, the decoder
// on all 254 finite codes.  Callers only encode quotients x / (amax / 448),
// whose magnitude stays below 449.8 even when the scale is an fp32 subnormal,
// so saturation never comes into play.

// Four fp32 values -> four codes, byte i holding the code of the i-th value.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);   // bytes 0, 1
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);         // bytes 2, 3
    return (uint32_t)v;
}

// Four codes (byte i = code i) -> four fp32 values (exact).
__device__ __forceinline__ void unpack4_e4m3(uint32_t w, float* f) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);   // bytes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);    // bytes 2, 3
    f[0] = lo[0];
    f[1] = lo[1];
    f[2] = hi[0];
    f[3] = hi[1];
}

// ---- wave helpers ---------------------------------------------------------------

// DPP move of v (row_mask / bank_mask select the lanes written; the others, and
// lanes whose source falls outside the row, read 0).
template <int Ctrl, int RowMask = 0xF, int BankMask = 0xF>
__device__ __forceinline__ int dpp_or_zero(int v) {
    return __builtin_amdgcn_update_dpp(0, v, Ctrl, RowMask, BankMask, true);
}

// Inclusive prefix sum over the 64 lanes of a wave: sums of the last 1..4
// lanes within each 16-lane row (row_shr 1, 2, 3), then row_shr 4 and 8 into
// the upper banks complete each row, and row_bcast15 / row_bcast31 carry rows
// into the next ones.  Seven DPP adds, no LDS traffic.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    int x = v;
    x += dpp_or_zero<0x111>(v);              // row_shr:1
    x += dpp_or_zero<0x112>(v);              // row_shr:2
    x += dpp_or_zero<0x113>(v);              // row_shr:3
    x += dpp_or_zero<0x114, 0xF, 0xE>(x);    // row_shr:4 into lanes 4..15 of each row
    x += dpp_or_zero<0x118, 0xF, 0xC>(x);    // row_shr:8 into lanes 8..15
    x += dpp_or_zero<0x142, 0xA>(x);         // row_bcast:15 into rows 1 and 3
    x += dpp_or_zero<0x143, 0xC>(x);         // row_bcast:31 into rows 2 and 3
    return x;
}

// Barrier for a block's LDS traffic only: orders its LDS accesses across the
// barrier without draining its outstanding global loads and stores, which a
// full __syncthreads (a workgroup release fence) waits for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Rank whose receive region holds receive row q: the number of region starts
// rank_recv_off[0..P] that are <= q, less one (a ballot per 64 ranks; the
// loads use clamped addresses, so loads the caller issued before stay in
// flight with them).
__device__ __forceinline__ int owner_rank(const int32_t* __restrict__ rank_recv_off, int P, int q) {
    const int lane = threadIdx.x & (kWave - 1);
    int count = 0;
    for (int r0 = 0; r0 <= P; r0 += kWave) {
        const int r = r0 + lane;
        const int start = rank_recv_off[min(r, P)];
        count += __popcll(__ballot(r <= P && start <= q));
    }
    return count - 1;
}

// Row and slice of this workgroup in a 1-D grid of rows x slices workgroups
// with the slices of a row adjacent (row_grid on the host).
struct RowSlice {
    int row, slice;
};
__device__ __forceinline__ RowSlice row_slice(int slices) {
    const int b = blockIdx.x;
    // one and two slices (rows up to 8 KiB, and up to 16 KiB) skip the integer division
    const int row = slices == 1 ? b : slices == 2 ? b >> 1 : b / slices;
    return {row, b - row * slices};
}

// Work item of this workgroup in a token-affine grid (TokenGrid on the host):
// token t, slot j and slice; false for the workgroups that pad a round to a
// power of two, and past the last token.
__device__ __forceinline__ bool token_item(int groups, int slices, int tpb_log2, int m_log2, int T, int& t, int& j,
                                           int& slice) {
    const int w = blockIdx.x;
    const int round = w >> m_log2, rem = w & ((1 << m_log2) - 1);
    if (rem >= groups * slices) return false;
    const int g = slices == 1 ? rem : slices == 2 ? rem >> 1 : rem / slices;
    slice = rem - g * slices;
    j = round >> tpb_log2;
    t = (g << tpb_log2) + (round & ((1 << tpb_log2) - 1));
    return t < T;
}

// Exclusive prefix sum over the block (blockDim.x <= 1024, a multiple of 64).
// `tmp` needs blockDim.x / 64 + 1 ints of LDS.  Every thread of the block must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int incl = wave_inclusive_scan(v);
    if (lane == kWave - 1) tmp[wave] = incl;
    lds_barrier();
    if (wave == 0) {
        int w = lane < nw ? tmp[lane] : 0;
        const int wincl = wave_inclusive_scan(w);
        if (lane < nw) tmp[lane] = wincl - w;
        if (lane == nw - 1) tmp[nw] = wincl;
    }
    lds_barrier();
    const int out = tmp[wave] + incl - v;
    if (total) *total = tmp[nw];
    lds_barrier();
    return out;
}

}  // namespace moe
