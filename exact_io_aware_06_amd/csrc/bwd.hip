// Attention backward, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// The attention matrix is recomputed from Q, K and the forward's LSE instead
// of being stored ("Quadratic Complexity Bottleneck", FlashAttention entry;
// "Chapter 3.1 - The Cost of Attention", section 5). With P = exp(S - LSE),
// S = scale Q K^T (masked), and D = rowsum(dO * O):
//
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
//   dK = scale dS^T Q.
//
// Three kernels, no atomics (every output element has exactly one writer, so
// results are deterministic):
//   bwd_dq    one work-group per (batch, head, 128 query rows), four waves of
//             32 rows; first D of its rows (from its dO and the stored O),
//             which it also publishes with the exp2-domain LSE for bwd_dkdv;
//             then, streaming the visible 64-key K/V tiles through LDS:
//             S^T = K Q^T and dP^T = V dO^T on matrix cores (Q, dO stay in
//             registers), dS^T on the vector ALU, then dQ^T += K^T dS^T with
//             dS^T straight from registers and K^T gathered by transposing LDS
//             reads. The same structure as the forward kernel.
//   bwd_dkdv  one work-group per (batch, query head, 128 keys), four waves of
//             32 keys; K stays in registers and V in LDS while 32-row Q / dO
//             tiles stream through LDS: S = Q K^T and dP = dO V^T, then
//             dV^T += dO^T P and dK^T += Q^T dS with P, dS straight from
//             registers. Each query head writes its own dK, dV (bf16 when the
//             K/V head has one query head, fp32 partials otherwise).
//   bwd_gsum  sums the fp32 partials over the G query heads of each K/V head
//             (GQA) and rounds to bf16.
// Splitting dK/dV work by query head keeps the causal work per work-group
// balanced enough (heaviest key tiles first) with no cross-work-group
// reduction other than the small group sum.
//
// Packed documents (the backward of the packed forward): the batch index is
// the document, whose rows are located through the row offsets; work-groups
// past a document's end exit at once, as in the forward.

#include <cstdio>

#include "common.hpp"
#include "launch.hpp"

namespace miattn {

namespace {

constexpr int kThreads = 256;

// An LDS tile of ROWS rows x D bf16, row-major, 16-byte chunks of each row
// XOR-swizzled, filled by 1 KB global-to-LDS blocks (64 lanes x 16 bytes).
template <int D, int ROWS>
struct LTile {
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int RPB = 64 / CPR;
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int NBLK = BYTES / 1024;
  static constexpr int BPW = NBLK / 4;
  static_assert(NBLK % 4 == 0, "DMA blocks split over four waves");
};

// The swizzle keeps both kinds of read free of bank conflicts on an LDS that
// serves 256 bytes (64 banks) per cycle: 16-byte operand reads of 16
// consecutive rows, and 8-byte transposing reads whose 32 lanes per cycle
// cover 4 rows (d = 128: the rows of an aligned group of four differ in the
// high swizzle bits; d = 64: rows r and r + 2 do).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Per-lane LDS byte offsets into such a tile.
//  row_off: matrix-core operand "row l32, k = 16 ks + 8 g .. + 8" (add
//           32 * rb * ROWB for row block rb).
//  tr_off:  transposing reads giving "column (dim) db*32 + l32, rows
//           16 tt + {4g..4g+3, 8+4g..8+4g+3}" (add 16 * tt * ROWB), the row
//           order the matrix-core result registers hold.
//  dma_off: this lane's slot in the wave's DMA blocks.
template <int D>
struct LOffsets {
  uint32_t row_off[D / 16];
  uint32_t tr_off[D / 32][2];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, g = lane >> 5;
    const int sw = swz<D>(l32);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      row_off[ks] = (uint32_t)(l32 * D * 2 + (((2 * ks + g) ^ sw) << 4));
    const int j = lane & 15, a = j & 3, e = j >> 2, hh = (lane >> 4) & 1;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int r = 4 * g + e + 8 * qh;
      const int rs = swz<D>(r);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int c = 4 * db + 2 * hh + (a >> 1);
        tr_off[db][qh] = (uint32_t)(r * D * 2 + ((c ^ rs) << 4) + (a & 1) * 8);
      }
    }
  }
};

template <int D, int ROWS>
__device__ __forceinline__ uint32_t dma_off(int wave, int lane, int i) {
  using T = LTile<D, ROWS>;
  const int blk = wave * T::BPW + i;
  const int r = blk * T::RPB + lane / T::CPR;
  return (uint32_t)(r * T::ROWB + (((lane % T::CPR) ^ swz<D>(r)) << 4));
}

// V^T-style operand: two transposing reads of an LDS tile.
__device__ __forceinline__ bf16x8 tr_operand(const lds_u8* tile, uint32_t o0, uint32_t o1) {
  const uint2 lo = lds_tr_b64(tile, o0);
  const uint2 hi = lds_tr_b64(tile, o1);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* delta;  // [B, H, Nq]
  float* lse2;   // [B, H, Nq]: LSE * log2(e), +inf where LSE = -inf
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dk_part;  // [B, H, Nk, d] when G > 1
  float* dv_part;
  int B, H, Hkv, Nq, Nk, G;
  float scale, scale_log2;
  int causal, window;
  int nqt, nkt;
  int xcd_remap;
  // Packed documents (null for fixed-length calls): B documents whose query
  // and key rows are [cu_q[b], cu_q[b+1]) and [cu_k[b], cu_k[b+1]) of packed
  // sequences of Nq and Nk rows.
  const int* cu_q;
  const int* cu_k;
};

// The rows one (batch or document, query head) works on: Nq queries from row
// head_q of Q / dO / dQ / LSE / D, Nk keys from row head_kv of K / V / dK /
// dV, and the fp32 dK / dV partials of this query head from row head_p. A
// document whose offsets are out of order or out of range has no rows.
struct Rows {
  int Nq, Nk;
  size_t head_q, head_kv, head_p;
};

__device__ __forceinline__ Rows rows_of(const BwdParams& p, int b, int h, int kvh) {
  Rows r;
  if (p.cu_q == nullptr) {
    r.Nq = p.Nq;
    r.Nk = p.Nk;
    r.head_q = (size_t)(b * p.H + h) * p.Nq;
    r.head_kv = (size_t)(b * p.Hkv + kvh) * p.Nk;
    r.head_p = (size_t)(b * p.H + h) * p.Nk;
  } else {
    const int qs = p.cu_q[b], qe = p.cu_q[b + 1];
    const int ks = p.cu_k[b], ke = p.cu_k[b + 1];
    const bool ok = 0 <= qs && qs <= qe && qe <= p.Nq && 0 <= ks && ks <= ke && ke <= p.Nk;
    r.Nq = ok ? qe - qs : 0;
    r.Nk = ok ? ke - ks : 0;
    r.head_q = (size_t)h * p.Nq + (ok ? qs : 0);
    r.head_kv = (size_t)kvh * p.Nk + (ok ? ks : 0);
    r.head_p = (size_t)h * p.Nk + (ok ? ks : 0);
  }
  return r;
}

// ---------------------------------------------------------------------------
// dQ.

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2)))
void bwd_dq_kernel(BwdParams p) {
  using KT = LTile<D, 64>;
  constexpr int BN = 64, KB = 2, KS = D / 16, DB = D / 32, PS = BN / 16;
  // K ring of two tiles at [0, 2 BYTES), V ring at [2 BYTES, 4 BYTES).
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * KT::BYTES];
  lds_u8* const L = lds_ptr(smem);
  constexpr int KRING = 0, VRING = 2 * KT::BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // Work-group -> (b, h, query tile): heaviest causal tiles first; with
  // (B * Hkv) % 8 == 0 the work-groups of one K/V head share one XCD.
  int b, h, qt;
  {
    const int id = blockIdx.x;
    if (p.xcd_remap) {
      const int xcd = id & 7, slot = id >> 3;
      const int per_rank = ((p.B * p.Hkv) >> 3) * p.G;
      const int rank = slot / per_rank, rem = slot - rank * per_rank;
      const int ul = rem / p.G, gh = rem - ul * p.G;
      const int u = ul * 8 + xcd;
      b = u / p.Hkv;
      h = (u - b * p.Hkv) * p.G + gh;
      qt = p.nqt - 1 - rank;
    } else {
      const int bh = p.B * p.H, rank = id / bh, rem = id - rank * bh;
      b = rem / p.H;
      h = rem - b * p.H;
      qt = p.nqt - 1 - rank;
    }
  }
  const int kvh = h / p.G;
  const Rows R = rows_of(p, b, h, kvh);
  const int Nq = R.Nq, Nk = R.Nk;
  const int q0 = qt * 128;
  if (q0 >= Nq) return;  // a query tile past the end of its document
  const int off = Nk - Nq;
  const int q_last = min(q0 + 128, Nq) - 1;
  const long long p_lo = (long long)q0 + off, p_hi = (long long)q_last + off;
  long long key_lo = 0, key_hi = Nk;
  if (p.causal) key_hi = min(key_hi, p_hi + 1);
  else if (p.window > 0) key_hi = min(key_hi, p_hi + p.window + 1);
  if (p.window > 0) key_lo = max(key_lo, p_lo - p.window);
  const int kt_lo = key_hi > key_lo ? (int)(key_lo / BN) : 0;
  const int kt_hi = key_hi > key_lo ? (int)((key_hi + BN - 1) / BN) : 0;
  const int ntiles = kt_hi - kt_lo;

  const int qrow = q0 + wave * 32 + l32;
  const bool qvalid = qrow < Nq;
  const long long qpos = (long long)qrow + off;
  const long long lo_q = p.window > 0 ? qpos - p.window : 0;
  long long hi_q = p.causal ? qpos : (p.window > 0 ? qpos + p.window : (long long)Nk - 1);
  hi_q = min(hi_q, (long long)Nk - 1);
  const size_t head_q = R.head_q;

  bf16x8 qf[KS], df[KS];
  float dlt = 0.f;  // D = rowsum(dO * O) of this row, fp32 over the stored bf16 O
  {
    const size_t r = (head_q + (qvalid ? qrow : 0)) * D + g * 8;
    bf16x8 of[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = as_bf16x8(load16(p.q + r + ks * 16, qvalid));
      df[ks] = as_bf16x8(load16(p.dout + r + ks * 16, qvalid));
      of[ks] = as_bf16x8(load16(p.o + r + ks * 16, qvalid));
    }
    // This lane holds half of the row's dims (chunks g, g + 2, ...), lane
    // l32 + 32 the other half.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) dlt = __builtin_fmaf((float)df[ks][i], (float)of[ks][i], dlt);
    dlt += swap_halves(dlt);
  }
  // exp2-domain LSE of this row (+inf for a row that sees no key, so every
  // P of it is 0). It and D are published for the dK / dV pass, which reads
  // them for rows of its documents only, all of which have a dQ work-group.
  const float lse_row = qvalid ? p.lse[head_q + qrow] : -kInf;
  const float lse2 = lse_row == -kInf ? kInf : lse_row * kLog2e;
  if (qvalid && g == 0) {
    p.delta[head_q + qrow] = dlt;
    p.lse2[head_q + qrow] = lse2;
  }

  LOffsets<D> lo;
  lo.init(lane);
  uint32_t doff[KT::BPW];
#pragma unroll
  for (int i = 0; i < KT::BPW; ++i) doff[i] = dma_off<D, 64>(wave, lane, i);

  const size_t head_kv = R.head_kv;
  const uint16_t* kbase = p.k + head_kv * D;
  const uint16_t* vbase = p.v + head_kv * D;

  // Key tiles needing no per-element mask for any row here: [full_lo, full_hi)
  // (inside the keys, at or before the first row's diagonal, at or after the
  // last row's window edge, within the first row's window when not causal).
  int full_lo, full_hi;
  {
    auto floor_div = [](long long a, long long b) { return a >= 0 ? a / b : -((-a + b - 1) / b); };
    long long fl = -1, fh = Nk / BN;
    if (p.window > 0) fl = -floor_div(p.window - p_hi, BN);  // ceil((p_hi - W) / BN)
    if (p.causal) fh = min(fh, floor_div(p_lo + 1, BN));
    if (p.window > 0 && !p.causal) fh = min(fh, floor_div(p_lo + p.window + 1, BN));
    full_lo = (int)max(fl, -1LL);
    full_hi = (int)max(min(fh, (long long)Nk / BN + 1), -1LL);
  }
  auto tile_partial = [&](int kt) -> bool { return !(kt >= full_lo && kt < full_hi); };

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  // K and V tile kt into ring slot `slot` (rows at or past Nk read as zero),
  // issued from inline assembly so that the LDS reads of the current tile do
  // not wait for it; the barrier at the end of the step is preceded by the
  // wait.
  auto issue_tile = [&](long long kt, int slot) {
    const long long r0 = kt * BN;
    const uint32_t bytes = r0 < Nk ? (uint32_t)((Nk - r0) * KT::ROWB) : 0u;
    const long long rr = r0 < Nk ? r0 : 0;
    const i32x4 rk = rsrc_words(kbase + rr * D, bytes);
    const i32x4 rv = rsrc_words(vbase + rr * D, bytes);
#pragma unroll
    for (int i = 0; i < KT::BPW; ++i) {
      dma16_async(rk, L + KRING + slot * KT::BYTES + (wave * KT::BPW + i) * 1024, doff[i]);
      dma16_async(rv, L + VRING + slot * KT::BYTES + (wave * KT::BPW + i) * 1024, doff[i]);
    }
  };
  if (ntiles > 0) {
    issue_tile(kt_lo, 0);
    wait_vmem();
    __syncthreads();
  }
  for (int t = 0; t < ntiles; ++t) {
    const int kt = kt_lo + t;
    const int slot = t & 1;
    // The next tile (an empty range after the last one) into the other slot.
    ring_fence_before_copy();
    issue_tile(t + 1 < ntiles ? kt + 1 : Nk / BN + 1, 1 - slot);
    ring_fence_after_copy();
    const lds_u8* kt_lds = L + KRING + slot * KT::BYTES;
    const lds_u8* vt_lds = L + VRING + slot * KT::BYTES;

    // S^T = K Q^T and dP^T = V dO^T (keys as rows, this wave's rows as columns),
    // software-pipelined by k-step: the K and V operands of step ks + 1 are
    // read while the 2 KB independent products of step ks issue.
    f32x16 s[KB], dp[KB];
    {
      bf16x8 ka[2][KB], vb[2][KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
        ka[0][kb] = lds_b128(kt_lds, lo.row_off[0] + kb * 32 * KT::ROWB);
        vb[0][kb] = lds_b128(vt_lds, lo.row_off[0] + kb * 32 * KT::ROWB);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          s[kb] = mfma32x32x16(ka[ks & 1][kb], qf[ks], s[kb]);
          if (ks + 1 < KS)
            ka[(ks + 1) & 1][kb] = lds_b128(kt_lds, lo.row_off[ks + 1] + kb * 32 * KT::ROWB);
          dp[kb] = mfma32x32x16(vb[ks & 1][kb], df[ks], dp[kb]);
          if (ks + 1 < KS)
            vb[(ks + 1) & 1][kb] = lds_b128(vt_lds, lo.row_off[ks + 1] + kb * 32 * KT::ROWB);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KB, 3);
#pragma unroll
      for (int i = 0; i < 2 * KB * KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
        if (i < 2 * KB * (KS - 1)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
      }
    }
    mfma_drain();

    if (tile_partial(kt)) {
      const long long base = (long long)kt * BN + 4 * g;
      const int rl = (int)max(min(lo_q - base, (long long)BN + 1), -1LL);
      const int rh = (int)max(min(hi_q - base, (long long)BN + 1), -1LL);
      const KeyRange vis(rl, rh);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
          s[kb][r] = vis.holds(c) ? s[kb][r] : -kInf;
        }
    }

    // dS^T = P^T * (dP^T - D), rounded to bf16 as the next product's operand.
    bf16x8 dsf[PS];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x8 ds;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pv = fast_exp2(__builtin_fmaf(s[kb][hf * 8 + i], p.scale_log2, -lse2));
          ds[i] = pv * (dp[kb][hf * 8 + i] - dlt);
        }
        dsf[kb * 2 + hf] = to_bf16x8(ds);
      }

    // dQ^T += K^T dS^T, software-pipelined by key step like the S^T products.
    {
      auto kread = [&](int db, int tt) {
        return tr_operand(kt_lds, lo.tr_off[db][0] + tt * 16 * KT::ROWB,
                          lo.tr_off[db][1] + tt * 16 * KT::ROWB);
      };
      bf16x8 kt_op[2][DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) kt_op[0][db] = kread(db, 0);
#pragma unroll
      for (int tt = 0; tt < PS; ++tt)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          acc[db] = mfma32x32x16(kt_op[tt & 1][db], dsf[tt], acc[db]);
          if (tt + 1 < PS) kt_op[(tt + 1) & 1][db] = kread(db, tt + 1);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 4);
#pragma unroll
      for (int i = 0; i < DB * PS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 4);
        if (i < DB * (PS - 1)) __builtin_amdgcn_sched_group_barrier(0x100, 2, 4);
      }
    }

    wait_vmem();
    __syncthreads();
  }
  mfma_drain();

  // dQ goes to device memory through LDS (store_rows_bf16), each wave's 32
  // rows in its own 64 D bytes of the K ring, which no wave reads after the
  // last step's barrier (and whose copies that barrier has seen land).
  {
    uint2 w[D / 8];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        w[db * 4 + rr].x = pack_bf16x2(acc[db][rr * 4 + 0] * p.scale, acc[db][rr * 4 + 1] * p.scale);
        w[db * 4 + rr].y = pack_bf16x2(acc[db][rr * 4 + 2] * p.scale, acc[db][rr * 4 + 3] * p.scale);
      }
    const int row0 = q0 + wave * 32;
    store_rows_bf16<D>(L + KRING + wave * 64 * D, w, lane_id(), p.dq + (head_q + row0) * D, Nq - row0);
  }
}

// ---------------------------------------------------------------------------
// dK, dV.

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(BwdParams p) {
  using QT = LTile<D, 32>;   // one 32-row Q (or dO) step
  using VT = LTile<D, 128>;  // the work-group's V tile
  constexpr int KS = D / 16, DB = D / 32;
  // LDS: V tile, then the Q ring (2 steps) and the dO ring (2 steps).
  __shared__ __attribute__((aligned(1024))) unsigned char smem[VT::BYTES + 4 * QT::BYTES];
  // [slot][lse2, D][row]: rows 32..63 of each line take the zeros of the
  // unused half of a 64-lane copy.
  __shared__ __attribute__((aligned(256))) float stat[2][2][64];
  lds_u8* const L = lds_ptr(smem);
  constexpr int VOFF = 0, QRING = VT::BYTES, DRING = VT::BYTES + 2 * QT::BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // Work-group -> (b, h, key tile): lowest key tiles (most visible query
  // rows under a causal mask) first; with (B * H) % 8 == 0 the work-groups
  // of one query head share one XCD (their Q / dO streams overlap).
  int b, h, kt;
  {
    const int id = blockIdx.x;
    const int bh = p.B * p.H;
    if (p.xcd_remap) {
      const int xcd = id & 7, slot = id >> 3;
      const int per_rank = bh >> 3;
      const int rank = slot / per_rank, ul = slot - rank * per_rank;
      const int u = ul * 8 + xcd;
      b = u / p.H;
      h = u - b * p.H;
      kt = rank;
    } else {
      const int rank = id / bh, rem = id - rank * bh;
      b = rem / p.H;
      h = rem - b * p.H;
      kt = rank;
    }
  }
  const int kvh = h / p.G;
  const Rows R = rows_of(p, b, h, kvh);
  const int Nq = R.Nq, Nk = R.Nk;
  const int k0 = kt * 128;
  if (k0 >= Nk) return;  // a key tile past the end of its document
  const int k1 = min(k0 + 127, Nk - 1);
  const int off = Nk - Nq;

  // Query rows that see any key of [k0, k1]; steps of 32 rows over them.
  long long i_lo = 0, i_hi = (long long)Nq - 1;
  if (p.causal) {
    i_lo = (long long)k0 - off;
    if (p.window > 0) i_hi = min(i_hi, (long long)k1 + p.window - off);
  } else if (p.window > 0) {
    i_lo = (long long)k0 - p.window - off;
    i_hi = min(i_hi, (long long)k1 + p.window - off);
  }
  i_lo = max(i_lo, 0LL);
  const int st_lo = i_hi >= i_lo ? (int)(i_lo / 32) : 0;
  const int nsteps = i_hi >= i_lo ? (int)(i_hi / 32) + 1 - st_lo : 0;

  // This lane's key and the query rows that see it: [jq_lo, jq_hi].
  const int key = k0 + wave * 32 + l32;
  const bool kvalid = key < Nk;
  long long jq_lo = 0, jq_hi = (long long)Nq - 1;
  if (p.causal) {
    jq_lo = (long long)key - off;
    if (p.window > 0) jq_hi = (long long)key + p.window - off;
  } else if (p.window > 0) {
    jq_lo = (long long)key - p.window - off;
    jq_hi = (long long)key + p.window - off;
  }

  const size_t head_kv = R.head_kv;
  const size_t head_q = R.head_q;
  // K as the B operand of S = Q K^T (k = dims), kept in registers.
  bf16x8 kf[KS];
  {
    const size_t r = (head_kv + (kvalid ? key : 0)) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = as_bf16x8(load16(p.k + r + ks * 16, kvalid));
  }

  LOffsets<D> lo;
  lo.init(lane);
  // The swizzle permutes 16-byte chunks by XOR, so the offset of k-step ks
  // is that of k-step 0 with (ks << 5) XORed in, and that of dim block db of
  // a transposing read is block 0's with (db << 6) XORed in.
  uint32_t rb = lo.row_off[0];
  uint32_t vb = lo.row_off[0] + wave * 32 * VT::ROWB;  // this wave's V rows
  uint32_t tb0 = lo.tr_off[0][0], tb1 = lo.tr_off[0][1];
  uint32_t qdoff[QT::BPW], vdoff[VT::BPW];
#pragma unroll
  for (int i = 0; i < QT::BPW; ++i) qdoff[i] = dma_off<D, 32>(wave, lane, i);
#pragma unroll
  for (int i = 0; i < VT::BPW; ++i) vdoff[i] = dma_off<D, 128>(wave, lane, i);

  const uint16_t* qbase = p.q + head_q * D;
  const uint16_t* dbase = p.dout + head_q * D;

  // Copies of step st's rows into ring slot `slot`: Q and dO rows by every
  // wave, the exp2-domain LSE and D by waves 0 and 1. Rows at or past Nq read
  // as zero; with their Q and dO rows zero they add nothing to dK or dV. The
  // copies are issued from inline assembly, so they run on while the LDS
  // reads of the current step proceed; the caller waits before the barrier
  // that publishes them.
  auto issue_step = [&](int st, int slot) {
    const long long r0 = (long long)st * 32;
    const uint32_t qbytes = r0 < Nq ? (uint32_t)((Nq - r0) * QT::ROWB) : 0u;
    const long long rr = r0 < Nq ? r0 : 0;
    const i32x4 rq = rsrc_words(qbase + rr * D, qbytes);
    const i32x4 rd = rsrc_words(dbase + rr * D, qbytes);
#pragma unroll
    for (int i = 0; i < QT::BPW; ++i) {
      dma16_async(rq, L + QRING + slot * QT::BYTES + (wave * QT::BPW + i) * 1024, qdoff[i]);
      dma16_async(rd, L + DRING + slot * QT::BYTES + (wave * QT::BPW + i) * 1024, qdoff[i]);
    }
    if (wave < 2) {
      const uint32_t sbytes = r0 < Nq ? (uint32_t)(min((long long)Nq - r0, 32LL) * 4) : 0u;
      const float* src = (wave == 0 ? p.lse2 : p.delta) + head_q + rr;
      dma4_async(rsrc_words(src, sbytes), lds_ptr(&stat[slot][wave][0]), (uint32_t)lane * 4u);
    }
  };
  // Does step st (rows [32 st, 32 st + 32)) need the per-element mask?
  auto step_partial = [&](int st) -> bool {
    const long long s0 = (long long)st * 32 + off, s1 = s0 + 31;  // positions
    if (p.causal) {
      if (s0 < k1) return true;
      if (p.window > 0 && s1 - p.window > k0) return true;
    } else if (p.window > 0) {
      if (s1 - p.window > k0 || s0 + p.window < k1) return true;
    }
    return false;
  };

  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dka[i] = f32x16{};
    dva[i] = f32x16{};
  }

  if (nsteps > 0) {
    {
      const uint32_t vbytes = k0 < Nk ? (uint32_t)((Nk - k0) * VT::ROWB) : 0u;
      const i32x4 rv = rsrc_words(p.v + (head_kv + k0) * D, vbytes);
#pragma unroll
      for (int i = 0; i < VT::BPW; ++i)
        dma16_async(rv, L + VOFF + (wave * VT::BPW + i) * 1024, vdoff[i]);
    }
    issue_step(st_lo, 0);
    wait_vmem();
    __syncthreads();
  }
  for (int t = 0; t < nsteps; ++t) {
    const int st = st_lo + t;
    const int slot = t & 1;
    // The next step's rows (an empty range after the last step), into the
    // other slot, whose previous contents the last barrier released.
    ring_fence_before_copy();
    issue_step(t + 1 < nsteps ? st + 1 : (Nq + 31) / 32 + 1, 1 - slot);
    ring_fence_after_copy();
    const lds_u8* q_lds = L + QRING + slot * QT::BYTES;
    const lds_u8* d_lds = L + DRING + slot * QT::BYTES;
    const lds_u8* v_lds = L + VOFF;

    // S = Q K^T and dP = dO V^T (query rows as rows, this wave's keys as
    // columns): lane (g, l32) holds key l32 for rows 8 c + 4 g + (0..3).
    // The bases are re-declared opaque each step so the compiler derives
    // the per-k-step offsets (an XOR each) instead of holding them all.
    asm volatile("" : "+v"(rb), "+v"(vb), "+v"(tb0), "+v"(tb1));
    // Operands of k-step ks + 1 are read while the products of ks issue.
    f32x16 s = f32x16{}, dp = f32x16{};
    bf16x8 qa = lds_b128(q_lds, rb), da = lds_b128(d_lds, rb), va = lds_b128(v_lds, vb);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 qn = qa, dn = da, vn = va;
      if (ks + 1 < KS) {
        qn = lds_b128(q_lds, rb ^ ((ks + 1) << 5));
        dn = lds_b128(d_lds, rb ^ ((ks + 1) << 5));
        vn = lds_b128(v_lds, vb ^ ((ks + 1) << 5));
      }
      s = mfma32x32x16(qa, kf[ks], s);
      dp = mfma32x32x16(da, va, dp);
      qa = qn;
      da = dn;
      va = vn;
    }
    // The first transposing operands of the dV / dK products (dim block 0)
    // are read beside the last products here and land during the softmax.
    auto tr_ops = [&](int db, bf16x8 (&od)[2], bf16x8 (&oq)[2]) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const uint32_t o0 = (tb0 ^ (db << 6)) + tt * 16 * QT::ROWB;
        const uint32_t o1 = (tb1 ^ (db << 6)) + tt * 16 * QT::ROWB;
        od[tt] = tr_operand(d_lds, o0, o1);
        oq[tt] = tr_operand(q_lds, o0, o1);
      }
    };
    bf16x8 od[2], oq[2];
    tr_ops(0, od, oq);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 5);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 5);
      if (i < 2 * (KS - 1)) {
        if (i & 1)
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 5);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 5);
      } else if (i == 2 * KS - 2) {
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 5);
      }
    }
    mfma_drain();

    if (step_partial(st)) {
      const long long base = (long long)st * 32 + 4 * g;  // row of register 0
      const int rl = (int)max(min(jq_lo - base, 33LL), -1LL);
      const int rh = (int)max(min(jq_hi - base, 33LL), -1LL);
      const KeyRange vis(rl, rh);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3);
        s[r] = vis.holds(c) ? s[r] : -kInf;
      }
    }

    // P and dS, rounded to bf16 as operands of the two products below.
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x8 pv, ds;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int c = hf * 2 + c2;  // rows 8 c + 4 g + (0..3)
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(&stat[slot][0][8 * c + 4 * g]);
        const f32x4 dl = *reinterpret_cast<const f32x4*>(&stat[slot][1][8 * c + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = c * 4 + e;
          const float pr = fast_exp2(__builtin_fmaf(s[r], p.scale_log2, -l2[e]));
          pv[c2 * 4 + e] = pr;
          ds[c2 * 4 + e] = pr * (dp[r] - dl[e]);
        }
      }
      pf[hf] = to_bf16x8(pv);
      dsf[hf] = to_bf16x8(ds);
    }

    // dV^T += dO^T P and dK^T += Q^T dS (dims as rows, keys as columns);
    // the operands of dim block db + 1 are read while db's products issue.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8 odn[2] = {od[0], od[1]}, oqn[2] = {oq[0], oq[1]};
      if (db + 1 < DB) tr_ops(db + 1, odn, oqn);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        dva[db] = mfma32x32x16(od[tt], pf[tt], dva[db]);
        dka[db] = mfma32x32x16(oq[tt], dsf[tt], dka[db]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        od[tt] = odn[tt];
        oq[tt] = oqn[tt];
      }
    }
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 6);
      if (i < 4 * (DB - 1)) __builtin_amdgcn_sched_group_barrier(0x100, 2, 6);
    }

    wait_vmem();
    __syncthreads();
  }
  mfma_drain();

  // Lane (g, l32) holds key `key`, dims db*32 + 8 rr + 4 g + (0..3). The
  // results go to device memory through LDS (store_rows_bf16 / _f32), each
  // wave's 32 keys in its own 128 D bytes of the V tile and the rings, which
  // no wave reads after the last step's barrier (and whose copies that
  // barrier has seen land); the fp32 partials pass through it one tensor
  // after the other.
  lds_u8* const region = L + wave * 128 * D;
  const int row0 = k0 + wave * 32;
  if (p.G == 1) {
    uint2 wk[D / 8], wv[D / 8];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int c = db * 4 + rr;
        wk[c].x = pack_bf16x2(dka[db][rr * 4 + 0] * p.scale, dka[db][rr * 4 + 1] * p.scale);
        wk[c].y = pack_bf16x2(dka[db][rr * 4 + 2] * p.scale, dka[db][rr * 4 + 3] * p.scale);
        wv[c].x = pack_bf16x2(dva[db][rr * 4 + 0], dva[db][rr * 4 + 1]);
        wv[c].y = pack_bf16x2(dva[db][rr * 4 + 2], dva[db][rr * 4 + 3]);
      }
    store_rows_bf16<D>(region, wk, lane, p.dk + (head_kv + row0) * D, Nk - row0);
    store_rows_bf16<D>(region + 64 * D, wv, lane, p.dv + (head_kv + row0) * D, Nk - row0);
  } else {
    f32x4 wk[D / 8], wv[D / 8];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = rr * 4;
        wk[db * 4 + rr] = f32x4{dka[db][r] * p.scale, dka[db][r + 1] * p.scale,
                                dka[db][r + 2] * p.scale, dka[db][r + 3] * p.scale};
        wv[db * 4 + rr] = f32x4{dva[db][r], dva[db][r + 1], dva[db][r + 2], dva[db][r + 3]};
      }
    const size_t part = (R.head_p + row0) * D;
    store_rows_f32<D>(region, wk, lane, p.dk_part + part, Nk - row0);
    store_rows_f32<D>(region, wv, lane, p.dv_part + part, Nk - row0);
  }
}

// ---------------------------------------------------------------------------
// GQA: dK, dV of a K/V head = sum over its G query heads' partials.

// One thread per 8 consecutive elements of a K/V head's dK and dV. The
// partials are read once, so they are loaded non-temporally; with G known at
// compile time every head's loads are issued before the first add. The sum
// runs over gh = 0 .. G-1 in that order either way.
template <int GC>
__global__ __launch_bounds__(kThreads) void bwd_gsum_kernel(BwdParams p, int d, long long n8) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;  // 8-element group
  if (i >= n8) return;
  const int G = GC > 0 ? GC : p.G;
  const long long per_head = (long long)p.Nk * d / 8;
  const long long bkv = i / per_head, rem = i - bkv * per_head;
  const long long b = bkv / p.Hkv, kvh = bkv - b * p.Hkv;
  const size_t head_stride = (size_t)p.Nk * d;
  const size_t src0 = ((size_t)(b * p.H + kvh * G) * p.Nk * d) + (size_t)rem * 8;
  const f32x4* kp = reinterpret_cast<const f32x4*>(p.dk_part + src0);
  const f32x4* vp = reinterpret_cast<const f32x4*>(p.dv_part + src0);
  const size_t hs4 = head_stride / 4;
  f32x8 sk = {}, sv = {};
  auto add = [&](f32x4 k0, f32x4 k1, f32x4 v0, f32x4 v1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sk[e] += k0[e];
      sk[e + 4] += k1[e];
      sv[e] += v0[e];
      sv[e + 4] += v1[e];
    }
  };
  if constexpr (GC > 0) {
    f32x4 k0[GC], k1[GC], v0[GC], v1[GC];
#pragma unroll
    for (int gh = 0; gh < GC; ++gh) {
      k0[gh] = __builtin_nontemporal_load(kp + gh * hs4);
      k1[gh] = __builtin_nontemporal_load(kp + gh * hs4 + 1);
      v0[gh] = __builtin_nontemporal_load(vp + gh * hs4);
      v1[gh] = __builtin_nontemporal_load(vp + gh * hs4 + 1);
    }
#pragma unroll
    for (int gh = 0; gh < GC; ++gh) add(k0[gh], k1[gh], v0[gh], v1[gh]);
  } else {
    for (int gh = 0; gh < G; ++gh)
      add(__builtin_nontemporal_load(kp + gh * hs4), __builtin_nontemporal_load(kp + gh * hs4 + 1),
          __builtin_nontemporal_load(vp + gh * hs4), __builtin_nontemporal_load(vp + gh * hs4 + 1));
  }
  const size_t dst = (size_t)i * 8;
  uint4 wk, wv;
  wk.x = pack_bf16x2(sk[0], sk[1]);
  wk.y = pack_bf16x2(sk[2], sk[3]);
  wk.z = pack_bf16x2(sk[4], sk[5]);
  wk.w = pack_bf16x2(sk[6], sk[7]);
  wv.x = pack_bf16x2(sv[0], sv[1]);
  wv.y = pack_bf16x2(sv[2], sv[3]);
  wv.z = pack_bf16x2(sv[4], sv[5]);
  wv.w = pack_bf16x2(sv[6], sv[7]);
  *reinterpret_cast<uint4*>(p.dk + dst) = wk;
  *reinterpret_cast<uint4*>(p.dv + dst) = wv;
}

template <int D>
hipError_t launch_bwd_d(BwdParams& prm, hipStream_t stream) {
  void* args[] = {&prm};
  hipError_t e = hipSuccess;
  // packed documents share one token axis per head: rows = H * total
  const long long nb = prm.cu_q != nullptr ? 1 : prm.B;
  const long long rows = nb * prm.H * prm.Nq;
  if (rows > 0) {
    // also writes D and the exp2-domain LSE of every row for the dK / dV pass
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<D>),
                        dim3((unsigned)((size_t)prm.B * prm.H * prm.nqt)), dim3(kThreads), args,
                        0, stream);
    if (e != hipSuccess) return e;
  }
  const size_t nkv = (size_t)prm.B * prm.H * prm.nkt;
  if (nkv == 0) return hipSuccess;
  // the dK / dV kernel groups work-groups by query head per XCD
  prm.xcd_remap = ((prm.B * prm.H) % 8 == 0) ? 1 : 0;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D>), dim3((unsigned)nkv),
                      dim3(kThreads), args, 0, stream);
  if (e != hipSuccess || prm.G == 1) return e;
  long long n8 = nb * prm.Hkv * prm.Nk * D / 8;
  int d = D;
  void* gargs[] = {&prm, &d, &n8};
  const void* gfn = prm.G == 2   ? reinterpret_cast<const void*>(&bwd_gsum_kernel<2>)
                    : prm.G == 4 ? reinterpret_cast<const void*>(&bwd_gsum_kernel<4>)
                    : prm.G == 8 ? reinterpret_cast<const void*>(&bwd_gsum_kernel<8>)
                                 : reinterpret_cast<const void*>(&bwd_gsum_kernel<0>);
  return hipLaunchKernel(gfn,
                         dim3((unsigned)((n8 + kThreads - 1) / kThreads)), dim3(kThreads), gargs,
                         0, stream);
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d) {
  const size_t delta = ((size_t)B * H * Nq * sizeof(float) + 255) / 256 * 256;
  const size_t part = (H / Hkv > 1) ? (size_t)B * H * Nk * d * sizeof(float) : 0;
  return 2 * delta + 2 * part;  // D, exp2-domain LSE, dK and dV partials
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<const uint16_t*>(a.o);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  const size_t nb = a.cu_q != nullptr ? 1 : (size_t)a.B;  // packed: one token axis
  const size_t delta = (nb * a.H * a.Nq * sizeof(float) + 255) / 256 * 256;
  p.delta = reinterpret_cast<float*>(ws);
  p.lse2 = reinterpret_cast<float*>(ws + delta);
  p.dk_part = reinterpret_cast<float*>(ws + 2 * delta);
  p.dv_part = p.dk_part + nb * a.H * a.Nk * a.d;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.B = a.B;
  p.H = a.H;
  p.Hkv = a.Hkv;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.G = a.H / a.Hkv;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  p.causal = a.causal;
  p.window = a.window;
  p.nqt = ((a.cu_q != nullptr ? a.max_q : a.Nq) + 127) / 128;
  p.nkt = ((a.cu_q != nullptr ? a.max_k : a.Nk) + 127) / 128;
  p.xcd_remap = ((a.B * a.Hkv) % 8 == 0) ? 1 : 0;
  if (log_enabled())
    fprintf(stderr, "[miattn] bwd d=%d dq_grid=%lld dkdv_grid=%lld G=%d\n", a.d,
            (long long)a.B * a.H * p.nqt, (long long)a.B * a.H * p.nkt, p.G);
  return a.d == 128 ? launch_bwd_d<128>(p, stream) : launch_bwd_d<64>(p, stream);
}

}  // namespace miattn
