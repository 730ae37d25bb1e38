// Device helpers shared by the libmiattn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kInf = __builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- LDS, buffer and DMA helpers -------------------------------------------

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ lds_u8* lds_ptr(void* shared_array) {
  return (lds_u8*)(shared_array);
}

// 16-byte LDS read at a byte offset.
__device__ __forceinline__ bf16x8 lds_b128(const lds_u8* base, uint32_t off) {
  return __builtin_bit_cast(bf16x8, *(const __attribute__((address_space(3))) uint4*)(base + off));
}

// Transposing LDS read of 16-bit elements. Within each group of 16 lanes,
// lane j names an 8-byte chunk (4 elements); lane i = 4a + c receives element
// c of the chunks named by lanes a, a + 4, a + 8 and a + 12, in that order.
__device__ __forceinline__ uint2 lds_tr_b64(const lds_u8* base, uint32_t off) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + off));
  return __builtin_bit_cast(uint2, r);
}

// 8-byte LDS store at a byte offset.
__device__ __forceinline__ void lds_st_b64(lds_u8* base, uint32_t off, uint2 v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  *(__attribute__((address_space(3))) u32x2*)(base + off) = u32x2{v.x, v.y};
}

// Raw buffer resource over [base, base + bytes): loads past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Global -> LDS copy of 16 bytes per lane: lane L's bytes at `voff` land at
// dst + 16 L. `dst` must be wave-uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, lds_u8* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, 0, 0, 0);
}

// The same copy issued from inline assembly, with the buffer descriptor as
// four SGPRs. The compiler does not see it as a memory operation, so it adds
// no wait before later LDS reads (it cannot prove that they touch another
// part of LDS and would otherwise wait for the copy to land). The caller
// waits itself (wait_vmem) before the data is read, and no compiler-issued
// LDS copy may be in flight across it (both use M0).
typedef int i32x4 __attribute__((ext_vector_type(4)));

// M0 is reserved for the compiler's own LDS copies; a kernel that uses these
// helpers issues all of its copies through them.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{(int)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (int)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
               (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

__device__ __forceinline__ void dma16_async(i32x4 rsrc, lds_u8* dst, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc)
               : "m0");
}

// 4 bytes per lane: lane L's dword at `voff` lands at dst + 4 L.
__device__ __forceinline__ void dma4_async(i32x4 rsrc, lds_u8* dst, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc)
               : "m0");
}

#pragma clang diagnostic pop

// s_waitcnt vmcnt(0): every vector-memory load of this wave (DMA included) done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Race-detector build. With MIATTN_SERIAL_RINGS=1 every copy into an LDS ring
// slot is fenced on both sides: a barrier before it (every wave has finished
// reading what the slot held) and, after it, a wait for this wave's copies
// and a barrier (every wave's copies have landed before anyone reads them).
// Each kernel also pads every matrix-core block whose results the vector ALU
// reads. The arithmetic and its order are unchanged, so this build must give
// bit-identical results to the pipelined one; a difference exposes a missing
// wait or barrier, or a too-short wait-state pad, in the pipelined kernels.
#ifndef MIATTN_SERIAL_RINGS
#define MIATTN_SERIAL_RINGS 0
#endif
constexpr bool kSerialRings = MIATTN_SERIAL_RINGS != 0;

__device__ __forceinline__ void ring_fence_before_copy() {
  if constexpr (kSerialRings) __syncthreads();
}
__device__ __forceinline__ void ring_fence_after_copy() {
  if constexpr (kSerialRings) {
    wait_vmem();
    __syncthreads();
  }
}

// 16-byte global load that yields zeros when `ok` is false.
__device__ __forceinline__ uint4 load16(const uint16_t* p, bool ok) {
  uint4 r = make_uint4(0u, 0u, 0u, 0u);
  if (ok) r = *reinterpret_cast<const uint4*>(p);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 lds_read_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// D += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate. Lane l holds
// A[l % 32][8 (l / 32) .. +8] and B[8 (l / 32) .. +8][l % 32]; D[i][j] sits in
// lane j + 32 * ((i / 4) % 2), register 4 (i / 8) + i % 4.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Pad between the last MFMA of a block and the first vector-ALU read of its
// result. With fp32 accumulators in arch VGPRs, this toolchain was seen to
// leave too few wait states after v_mfma_f32_32x32x16_bf16 on some control
// paths, so stale accumulator values were read back (wrong, run-to-run varying
// results). 24 explicit wait states, fenced against rescheduling, remove that
// and cost ~24 issue cycles per block, during which other waves issue.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of `x` in the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// max(x, x of the lane 32 away) with v_permlane32_swap (no LDS round trip):
// the swap of a register with itself returns, in its two results, this lane's
// value and its partner's, in an order that max() does not care about.
__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

// Boundary-tile masks test a compile-time key offset c >= 0 against a row's
// clamped bounds, rl <= c <= rh. As one unsigned comparison:
// c + neg_rl <= span with neg_rl = -rl and span = rh - rl, and for a row that
// sees no key here (rh < rl) c + 1 <= 0, false for every c. The two values are
// made opaque to the compiler, which would otherwise fold the clamped bounds
// back into two 64-bit comparisons per score.
struct KeyRange {
  unsigned neg_rl, span;
  __device__ __forceinline__ KeyRange(int rl, int rh) {
    const bool none = rh < rl;
    neg_rl = none ? 1u : (unsigned)(-rl);
    span = none ? 0u : (unsigned)(rh - rl);
    asm volatile("" : "+v"(neg_rl), "+v"(span));
  }
  __device__ __forceinline__ bool holds(int c) const { return (unsigned)c + neg_rl <= span; }
};

// Eight fp32 values to bf16, round to nearest even.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x8 v) {
  return __builtin_convertvector(v, bf16x8);
}

// Pairwise sum of eight fp32 values.
__device__ __forceinline__ float sum_f32x8(const f32x8 v) {
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

// Sum of the eight bf16 values in `v`, added to `acc` in fp32 (packed bf16
// dot products against (1, 1); the products are exact).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// ---- Row stores through LDS -------------------------------------------------
//
// A wave's 32 x D block of matrix-core results has lane l holding values
// 32 db + 8 rr + 4 (l / 32) .. + 4 of row l % 32 (db < D / 32, rr < 4).
// Stored straight from the registers, each instruction writes short pieces of
// 32 rows. These helpers move the block through a wave-private LDS region
// first, so that each store to device memory moves 16 contiguous bytes per
// lane and whole rows per instruction. In the region, row r sits at
// r * (row bytes) with its 16-byte chunks permuted by an XOR of r's low bits
// (for bf16 the two 8-byte halves of a chunk are also swapped when bit 4 of r
// is set). That puts the pieces written by each group of 32 lanes (8-byte,
// bf16) or 16 lanes (16-byte, fp32), and the chunks read by each group of 16
// lanes, on distinct banks; the counters still show a few conflict cycles
// per work-group, about 0.1 % of its time. The caller guarantees that no
// other wave touches the region
// until this wave is done with it. `out` is row 0 of the block; rows at or
// past `nrows` are not stored.

// This lane's index in its wave, from the lane counter (for code after a
// loop that has no register to spare for keeping it).
__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Orders this wave's LDS accesses on either side. One wave's LDS operations
// are performed in order, so this only keeps the compiler from moving them.
__device__ __forceinline__ void region_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// bf16 rows of D elements (64 D bytes of LDS); w[4 db + rr] holds the lane's
// four values as two packed pairs.
template <int D>
__device__ __forceinline__ void store_rows_bf16(lds_u8* region, const uint2 (&w)[D / 8], int lane,
                                                uint16_t* out, int nrows) {
  constexpr int ROWB = 2 * D, CPR = ROWB / 16, RPI = 64 / CPR;
  auto fsw = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  region_fence();  // after this wave's earlier reads of the region
  {
    const int r = lane & 31, g = lane >> 5;
    const uint32_t rb = (uint32_t)(r * ROWB + 8 * ((g ^ (r >> 4)) & 1));
#pragma unroll
    for (int c = 0; c < D / 8; ++c) lds_st_b64(region, rb + (uint32_t)((c ^ fsw(r)) << 4), w[c]);
  }
  region_fence();  // each lane reads back what other lanes of its wave wrote
  const int cl = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR;
    const uint32_t at = (uint32_t)(r * ROWB + ((cl ^ fsw(r)) << 4));
    const uint4 u = __builtin_bit_cast(uint4, lds_b128(region, at));
    const bool hi_first = (i * RPI) & 16;  // bit 4 of r, the same for every lane here
    const uint4 v = hi_first ? make_uint4(u.z, u.w, u.x, u.y) : u;
    if (r < nrows) *reinterpret_cast<uint4*>(out + (size_t)r * D + cl * 8) = v;
  }
}

// fp32 rows of D elements (128 D bytes of LDS); w[4 db + rr] holds the lane's
// four values.
template <int D>
__device__ __forceinline__ void store_rows_f32(lds_u8* region, const f32x4 (&w)[D / 8], int lane,
                                               float* out, int nrows) {
  constexpr int ROWB = 4 * D, CPR = ROWB / 16, RPI = 64 / CPR;
  region_fence();
  {
    const int r = lane & 31, g = lane >> 5;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const int chunk = 2 * c + g;  // 16-byte chunk of values 4 chunk .. + 4
      *(__attribute__((address_space(3))) f32x4*)(region + r * ROWB + ((chunk ^ (r & 15)) << 4)) =
          w[c];
    }
  }
  region_fence();
  const int cl = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR;
    const f32x4 v =
        *(const __attribute__((address_space(3))) f32x4*)(region + r * ROWB + ((cl ^ (r & 15)) << 4));
    if (r < nrows) *reinterpret_cast<f32x4*>(out + (size_t)r * D + cl * 4) = v;
  }
}

// Interleave the low halves (pick = 0) or high halves (pick = 1) of two
// dwords holding bf16 pairs: result = {a.half, b.half}.
__device__ __forceinline__ uint32_t interleave16(uint32_t a, uint32_t b, int pick) {
  return pick ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

__device__ __forceinline__ uint32_t u4_get(const uint4& u, int i) {
  return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

}  // namespace miattn
