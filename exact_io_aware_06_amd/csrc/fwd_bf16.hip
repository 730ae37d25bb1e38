// Fused attention forward, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// One work-group owns BM = 128 query rows of one (batch, head); each of its
// four waves owns 32 of those rows. The work-group streams the K/V tiles its
// rows can see through LDS and keeps everything else in registers: the
// score tile, the running row maximum and sum, and the output accumulator.
// Nothing of size Nq x Nk is ever written to device memory ("Quadratic
// Complexity Bottleneck", FlashAttention entry; grasp.study
// efficient-attention lesson, "Tiling and Kernel Fusion", "Online Softmax").
//
// Matrix-core formulation. With v_mfma_f32_32x32x16_bf16 a lane holds one
// column of the 32x32 result. The kernel therefore computes the transposed
// score tile S^T = K Q^T (keys as rows, this wave's 32 queries as columns):
// each lane then holds 16 keys of ONE query row, and the other 16 keys of
// that row sit in the lane 32 apart. The row max and row sum are in-lane
// reductions plus a single exchange between the two wave halves. The same
// registers, rounded to bf16, are directly the B operand of O^T += V^T P^T,
// so P never leaves the registers. K and V tiles are copied row-major from
// device memory into LDS by direct global-to-LDS loads; each lane gathers its
// V^T operand from the row-major V tile with two transposing LDS reads
// (ds_read_b64_tr_b16), in the key order its P registers hold.
//
// Online softmax (the pages' running max and running denominator, rescaling
// the partial output when the maximum grows) is done lazily: the reference
// maximum used for the exponentials is only moved when P would exceed 2^8,
// and it is then set 2^24 above the new maximum (exp2 domain). The final
// O / l and LSE = m + ln l are identical in exact arithmetic for any
// reference value, and in floating point P keeps its relative precision at
// any magnitude (only terms below ~2^-100 of the row maximum underflow).
// Bounding the growth keeps P <= 256, far from fp32/bf16 overflow; the
// headroom lets a row's maximum grow by 2^32 before the partial output has to
// be rescaled, which skips most of the rescaling multiplies. At d = 128 (bf16)
// the test needs no per-tile maximum: each lane's share of a tile's row sum
// bounds its P values, so a tile is accepted when that share is at most 2^8
// and otherwise (rarely) redone against a new reference. The d = 64 and fp8
// kernels take each tile's row maximum and compare it with the reference.
//
// Packed documents ("What Lost, and Why", closing section: the mask restarts
// at every document boundary) reuse the same kernel: the batch index becomes
// the document index, whose query and key rows are located through row
// offsets, and each document is masked as a sequence of its own. The grid
// then covers ceil(max document length / BM) query tiles per document and the
// tiles past a document's end exit at once.
//
// Work decomposition: grid = B * H * ceil(Nq / BM) work-groups, the query
// tiles with the most visible keys first (causal), and when (B * Hkv) is a
// multiple of 8 the work-groups of one K/V head are kept on one XCD (one L2)
// by undoing the round-robin dispatch of consecutive work-group ids across the
// eight XCDs. Key tiles that the causal or window mask hides from every row
// of the work-group are never loaded; only tiles that straddle a mask edge
// (or the end of the keys) evaluate the mask per element.

#include <cmath>
#include <cstdio>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace miattn {

namespace {

constexpr int kBM = 128;
constexpr int kThreads = 256;
// exp2-domain head-room before the reference maximum is moved.
constexpr float kRescaleThreshold = 8.0f;
// exp2-domain headroom above a row's new maximum when the reference moves.
constexpr float kRescaleHeadroom = 24.0f;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, H, Hkv, Nq, Nk, G;
  float scale;       // softmax scale on q.k
  float scale_log2;  // scale * log2(e)
  float thr_raw;     // kRescaleThreshold / scale_log2, in q.k units
  float head_raw;    // kRescaleHeadroom / scale_log2, in q.k units (0 if not finite)
  int causal, window;
  int nqt;
  int xcd_remap;
  int* counts;
  const int* cu_q;  // packed documents: row offsets, or null
  const int* cu_k;
};

template <int D, bool FP8 = false>
struct Tile {
  static constexpr int BN = 64;                      // keys per K/V tile
  static constexpr int ROWB = D * 2;                 // bytes per V row (and bf16 K row)
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int RPB = 64 / CPR;               // rows per 1 KB DMA block
  static constexpr int TILE = BN * ROWB;             // bytes of one V (or bf16 K) tile
  static constexpr int NBLK = TILE / 1024;           // DMA blocks per tile and tensor
  static constexpr int BPW = NBLK / 4;               // ... per wave
  static constexpr int KB = BN / 32;                 // 32-key blocks per tile
  static constexpr int DB = D / 32;                  // 32-dim blocks of O
  static constexpr int KS = D / 16;                  // k-steps of Q K^T (bf16)
  static constexpr int PS = BN / 16;                 // k-steps of P V
  // K tile: bf16, or fp8 e4m3 (one byte per element) for the fp8 Q K^T.
  static constexpr int KROWB = FP8 ? D : D * 2;
  static constexpr int KCPR = KROWB / 16;
  static constexpr int KRPB = 64 / KCPR;
  static constexpr int KTILE = BN * KROWB;
  static constexpr int KBPW = KTILE / 1024 / 4;
  static constexpr int KS8 = D / 64;                 // k-steps of the fp8 Q K^T
  static constexpr int LDS = 2 * KTILE + 2 * TILE;   // K ring + V ring
  static_assert(NBLK % 4 == 0 && (KTILE / 1024) % 4 == 0, "DMA blocks split over four waves");
};

// LDS layout of a K or V tile: row-major [key][d] with the 16-byte chunks of
// each row permuted by an XOR swizzle. The LDS serves 256 bytes (64 banks)
// per cycle: 16 lanes of a 16-byte read, 32 lanes of an 8-byte read. The
// swizzle keeps both reads free of bank conflicts: the 16 lanes reading one
// chunk of 16 consecutive rows (Q K^T operand) get 16 different chunk slots,
// and the 32 lanes of a transposing V^T read (4 rows x 2 chunks x 2 halves,
// for each of 2 x 2 lane groups) get 64 different banks, because the rows of
// an aligned group of four differ in the high bits of their swizzle (d = 128;
// for d = 64, two rows share a 256-byte bank line and rows r, r + 2 differ).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// The same for K rows of KROWB bytes (fp8 K: 128- or 64-byte rows).
template <int KROWB>
__device__ __forceinline__ int swzk(int r) {
  if (KROWB == 256) return ((r & 7) << 1) | ((r >> 3) & 1);
  if (KROWB == 128) return (r >> 1) & 7;
  return (r >> 2) & 3;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// D += A(32x64) * B(64x32), fp8 e4m3 inputs, fp32 accumulate; lane l holds
// 32 bytes of row l % 32 of A and of column l % 32 of B, for the same
// 32 values of k (chosen by l / 32); D as for the 32x32x16 products.
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // E8M0 block scales of 2^0 (exponent 127) on both operands
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 cat_u4(uint4 lo, uint4 hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ void decode_workgroup(const FwdParams& p, int id, int& b, int& h,
                                                 int& qt) {
  if (p.xcd_remap) {
    const int xcd = id & 7, slot = id >> 3;
    const int units = (p.B * p.Hkv) >> 3;  // (batch, kv-head) units per XCD
    const int per_rank = units * p.G;
    const int rank = slot / per_rank;
    const int rem = slot - rank * per_rank;
    const int ul = rem / p.G, gh = rem - ul * p.G;
    const int u = ul * 8 + xcd;
    b = u / p.Hkv;
    const int kvh = u - b * p.Hkv;
    h = kvh * p.G + gh;
    qt = p.nqt - 1 - rank;
  } else {
    const int bh = p.B * p.H;
    const int rank = id / bh;
    const int rem = id - rank * bh;
    b = rem / p.H;
    h = rem - b * p.H;
    qt = p.nqt - 1 - rank;
  }
}

// CAUSAL0: causal with no window, where only the diagonal bound can mask a key.
template <int D, bool COUNT, bool FP8 = false, bool CAUSAL0 = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 64 && !FP8 ? 3 : 2)))
void fwd_bf16_kernel(FwdParams p) {
  using T = Tile<D, FP8>;
  constexpr int BN = T::BN;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[T::LDS];
  lds_u8* const L = lds_ptr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  int b, h, qt;
  decode_workgroup(p, blockIdx.x, b, h, qt);
  const int kvh = h / p.G;
  const int q0 = qt * kBM;

  // Rows of this (batch, head): Nq queries from row head_q, Nk keys from row
  // head_kv. For packed documents b is the document, whose rows start at its
  // offsets within each head's packed sequence; a document whose offsets are
  // out of order or out of range is treated as empty.
  int Nq = p.Nq, Nk = p.Nk;
  size_t head_q = (size_t)(b * p.H + h) * p.Nq;
  size_t head_kv = (size_t)(b * p.Hkv + kvh) * p.Nk;
  if (p.cu_q != nullptr) {
    const int qs = p.cu_q[b], qe = p.cu_q[b + 1];
    const int ks = p.cu_k[b], ke = p.cu_k[b + 1];
    const bool ok = 0 <= qs && qs <= qe && qe <= p.Nq && 0 <= ks && ks <= ke && ke <= p.Nk;
    Nq = ok ? qe - qs : 0;
    Nk = ok ? ke - ks : 0;
    head_q = (size_t)h * p.Nq + (ok ? qs : 0);
    head_kv = (size_t)kvh * p.Nk + (ok ? ks : 0);
  }
  if (q0 >= Nq) {  // a query tile past the end of its document: nothing to do
    if (COUNT && threadIdx.x == 0) {
      int* c = p.counts + 2 * ((size_t)(b * p.H + h) * p.nqt + qt);
      c[0] = 0;
      c[1] = 0;
    }
    return;
  }
  const int off = Nk - Nq;
  const int q_last = min(q0 + kBM, Nq) - 1;
  const long long p_lo = (long long)q0 + off, p_hi = (long long)q_last + off;

  // Key range visible to any row of this work-group.
  long long key_lo = 0, key_hi = Nk;  // [key_lo, key_hi)
  if (p.causal) key_hi = min(key_hi, p_hi + 1);
  else if (p.window > 0) key_hi = min(key_hi, p_hi + p.window + 1);
  if (p.window > 0) key_lo = max(key_lo, p_lo - p.window);
  const int kt_lo = key_hi > key_lo ? (int)(key_lo / BN) : 0;
  const int kt_hi = key_hi > key_lo ? (int)((key_hi + BN - 1) / BN) : 0;
  const int ntiles = kt_hi - kt_lo;

  // This lane's query row and its Q fragments (B operand of S^T = K Q^T).
  const int qrow = q0 + wave * 32 + l32;
  const bool qvalid = qrow < Nq;
  const long long qpos = (long long)qrow + off;
  // Keys this row may see: [lo_q, hi_q] (used on boundary tiles only).
  const long long lo_q = p.window > 0 ? qpos - p.window : 0;
  long long hi_q = p.causal ? qpos : (p.window > 0 ? qpos + p.window : (long long)Nk - 1);
  hi_q = min(hi_q, (long long)Nk - 1);
  // The same bounds in 32 bits, clamped to [-2 BN, Nk + 2 BN]: a visited key
  // tile starts in [0, Nk), so every bound relative to it clamps to the same
  // value in [-1, BN + 1] as the unclamped one.
  const int lo_c = (int)max(min(lo_q, (long long)Nk + 2 * BN), -2LL * BN);
  const int hi_c = (int)max(min(hi_q, (long long)Nk + 2 * BN), -2LL * BN);
  bf16x8 qf[FP8 ? 1 : T::KS];
  i32x8 qf8[FP8 ? T::KS8 : 1];
  if constexpr (FP8) {
    // fp8 rows of D bytes, addressed as uint16 pairs: bytes 64 ks + 32 g .. + 32
    const uint16_t* qp = p.q + (head_q + (qvalid ? qrow : 0)) * (D / 2) + g * 16;
#pragma unroll
    for (int ks = 0; ks < T::KS8; ++ks)
      qf8[ks] = cat_u4(load16(qp + ks * 32, qvalid), load16(qp + ks * 32 + 8, qvalid));
  } else {
    const uint16_t* qp = p.q + (head_q + (qvalid ? qrow : 0)) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) qf[ks] = as_bf16x8(load16(qp + ks * 16, qvalid));
  }

  // LDS: K ring of two tiles at [0, 2 TILE), V ring of two tiles at
  // [2 TILE, 4 TILE). K runs two tiles ahead of the softmax, V one tile.
  constexpr int KRING = 0, VRING = 2 * T::KTILE;

  // Per-lane LDS byte offsets, fixed for the whole kernel.
  // Q K^T operand: row kb*32 + l32, chunk 2 ks + g.
  uint32_t koff[FP8 ? 1 : T::KS];
  uint32_t koff8[FP8 ? T::KS8 : 1][2];
  if constexpr (FP8) {
    // fp8: row kb*32 + l32, chunks 4 ks + 2 g and 4 ks + 2 g + 1
    const int sw = swzk<T::KROWB>(l32);
#pragma unroll
    for (int ks = 0; ks < T::KS8; ++ks)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        koff8[ks][hh] = (uint32_t)(l32 * T::KROWB + (((4 * ks + 2 * g + hh) ^ sw) << 4));
  } else {
    const int sw = swz<D>(l32);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks)
      koff[ks] = (uint32_t)(l32 * T::ROWB + (((2 * ks + g) ^ sw) << 4));
  }
  // V^T operand via transposing reads: as a source lane of its 16-lane group,
  // this lane names rows 4g + e (+8 for the second read) and dims
  // db*32 + 16h + 4a' of each 16-key step; lane 16h + i then receives dims
  // 16h + i of keys 4g..4g+3 (first read) and 8+4g..8+4g+3 (second read),
  // exactly the keys its P registers hold.
  uint32_t voff[T::DB][2];
  {
    const int j = lane & 15, a = j & 3, e = j >> 2, hh = (lane >> 4) & 1;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int r = 4 * g + e + 8 * qh;
      const int sw = swz<D>(r);
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const int c = 4 * db + 2 * hh + (a >> 1);
        voff[db][qh] = (uint32_t)(r * T::ROWB + ((c ^ sw) << 4) + (a & 1) * 8);
      }
    }
  }
  // DMA: block blk of a tile holds rows blk*RPB .. +RPB; lane L moves chunk
  // (L % CPR) ^ swz(row) of row blk*RPB + L / CPR into LDS slot L.
  uint32_t dvoff[T::BPW];
#pragma unroll
  for (int i = 0; i < T::BPW; ++i) {
    const int blk = wave * T::BPW + i;
    const int r = blk * T::RPB + lane / T::CPR;
    dvoff[i] = (uint32_t)(r * T::ROWB + (((lane % T::CPR) ^ swz<D>(r)) << 4));
  }
  // K tiles have their own geometry when K is fp8.
  uint32_t dkoff[T::KBPW];
#pragma unroll
  for (int i = 0; i < T::KBPW; ++i) {
    const int blk = wave * T::KBPW + i;
    const int r = blk * T::KRPB + lane / T::KCPR;
    dkoff[i] = FP8 ? (uint32_t)(r * T::KROWB + (((lane % T::KCPR) ^ swzk<T::KROWB>(r)) << 4))
                   : dvoff[i];
  }

  const uint16_t* kbase = p.k + head_kv * (T::KROWB / 2);  // uint16 units
  const uint16_t* vbase = p.v + head_kv * D;
  int loaded = 0, masked = 0;

  // DMA of one K (or V) tile kt into the LDS slot at byte `slot`.
  auto issue = [&](const uint16_t* base, int kt, int slot) {
    const long long k0 = (long long)kt * BN;
    const uint32_t bytes = k0 < Nk ? (uint32_t)((Nk - k0) * T::ROWB) : 0u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0 * D, bytes);
#pragma unroll
    for (int i = 0; i < T::BPW; ++i) dma16(rs, L + slot + (wave * T::BPW + i) * 1024, dvoff[i]);
  };
  // DMA of one K tile (bf16 or fp8 rows).
  auto issue_k = [&](int kt, int slot) {
    const long long k0 = (long long)kt * BN;
    const uint32_t bytes = k0 < Nk ? (uint32_t)((Nk - k0) * T::KROWB) : 0u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(kbase + k0 * (T::KROWB / 2), bytes);
#pragma unroll
    for (int i = 0; i < T::KBPW; ++i)
      dma16(rs, L + slot + (wave * T::KBPW + i) * 1024, dkoff[i]);
  };

  // Key tiles that need no per-element mask for any row here form one range
  // [full_lo, full_hi): a tile is full iff it lies inside the keys, ends at or
  // before the first row's diagonal (causal), starts at or after the last
  // row's window edge, and (non-causal window) ends within the first row's
  // window. Computed once; clamped to the tile indices a work-group visits.
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
  // Does key tile kt need the per-element mask for any valid row here?
  auto tile_partial = [&](int kt) -> bool { return !(kt >= full_lo && kt < full_hi); };

  f32x16 oacc[T::DB];
#pragma unroll
  for (int i = 0; i < T::DB; ++i) oacc[i] = f32x16{};
  float m_ref = -kInf;  // reference row maximum, q.k units
  // This lane's share of the row sum, twice: l_b sums the bf16-rounded P that
  // multiply V (so the weights O is normalised by sum to one exactly), l_f the
  // fp32 P (for an LSE as accurate as fp32 allows).
  float l_b = 0.f, l_f = 0.f;

  // S^T = K Q^T of the K tile in ring slot kslot.
  auto qk = [&](int kslot, f32x16 (&sacc)[T::KB]) {
    const lds_u8* kt_lds = L + KRING + kslot * T::KTILE;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
      sacc[kb] = f32x16{};
      if constexpr (FP8) {
#pragma unroll
        for (int ks = 0; ks < T::KS8; ++ks) {
          const uint32_t o = kb * 32 * T::KROWB;
          const i32x8 a = cat_u4(
              __builtin_bit_cast(uint4, lds_b128(kt_lds, koff8[ks][0] + o)),
              __builtin_bit_cast(uint4, lds_b128(kt_lds, koff8[ks][1] + o)));
          sacc[kb] = mfma32x32x64_fp8(a, qf8[ks], sacc[kb]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks)
          sacc[kb] =
              mfma32x32x16(lds_b128(kt_lds, koff[ks] + kb * 32 * T::ROWB), qf[ks], sacc[kb]);
      }
    }
  };

  // Boundary-tile mask, then this wave's row maxima of a score tile: returns
  // the candidate reference max and whether it must replace m_ref.
  auto mask_tile = [&](int kt, f32x16 (&sacc)[T::KB]) {
    // Key kt*BN + c + 4g is visible iff lo_q <= key <= hi_q; compare the
    // compile-time offset c against the row's bounds relative to the tile,
    // clamped to [-1, BN + 1].
    const int base = kt * BN + 4 * g;
    int rl = min(max(lo_c - base, -1), BN + 1);
    int rh = min(max(hi_c - base, -1), BN + 1);
    asm volatile("" : "+v"(rl), "+v"(rh));  // keep the comparisons in 32 bits
    auto apply = [&](auto vis) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
          sacc[kb][r] = vis(c) ? sacc[kb][r] : -kInf;
        }
    };
    if constexpr (CAUSAL0) {
      // Causal without a window: every row sees keys from 0, so rl <= 0 <= c
      // and one comparison per score against the diagonal bound decides (a
      // row with no key in this tile has rh = -1).
      apply([&](int c) { return c <= rh; });
    } else {
      const KeyRange vis(rl, rh);
      apply([&](int c) { return vis.holds(c); });
    }
  };
  auto row_max = [&](const f32x16 (&sacc)[T::KB]) -> float {
    float mx = -kInf;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    return max_halves(mx);
  };
  // Tile-sum overflow check instead of a per-tile row maximum (bf16, d = 128;
  // the fp8 kernel computes half of its softmax in block B, and at d = 64 the
  // redo path costs register spills, so both keep the per-tile maximum). A
  // lane's share of a tile's row sum bounds each of its P values, so
  // accepting tiles whose share is at most 2^8 keeps every P at or below 2^8,
  // the same bound the maximum-based test gives.
  constexpr bool kSumCheck = !FP8 && D == 128;
  constexpr float kSumLimit = 256.0f;
  // Move the reference maximum (and rescale O and the sums) if the new
  // tile's maximum exceeds it by more than the threshold.
  auto rescale = [&](float mx) {
    const float m_new = fmaxf(m_ref, mx);
    const bool need = m_new > m_ref + p.thr_raw;
    if (wave_any(need)) {
      mfma_drain();  // O was last written by matrix-core instructions
      const float m_up = m_new + p.head_raw;
      const float m_set = __builtin_isfinite(m_up) ? m_up : m_new;
      const float alpha = need ? fast_exp2((m_ref - m_set) * p.scale_log2) : 1.f;
      if (need) m_ref = m_set;
      l_b *= alpha;
      l_f *= alpha;
#pragma unroll
      for (int i = 0; i < T::DB; ++i) oacc[i] *= alpha;
    }
  };

  // One pipelined step for key tile t, whose scores s_cur are already masked
  // and whose maximum is already folded into m_ref:
  //   DMA K(t+2), V(t+1);
  //   block A: Q K^T of tile t+1 (matrix cores) beside exp / convert / sums of
  //            tile t (vector ALU);
  //   block B: O += P V of tile t beside mask and row max of tile t+1;
  //   barrier, then the (rare) rescale for tile t+1.
  // K(t+1) sits in ring slot kslot_next, V(t) in ring slot vslot; MASK_NEXT
  // selects the boundary-tile variant of block B. The work-group's last step
  // (LAST, a compile-time tag) has no next tile: its block A is the softmax
  // alone and block B the P V products alone.
  auto step = [&](auto last_tag, int t, int kslot_next, int vslot, f32x16 (&s_cur)[T::KB],
                  f32x16 (&s_nxt)[T::KB], bool mask_next) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int kt = kt_lo + t;
    if (COUNT && t + 2 < ntiles) ++loaded;
    float msub = (m_ref == -kInf) ? 0.f : m_ref * p.scale_log2;

    // P = exp2(S scale_log2 - msub) of the 32-key blocks [kb0, kb1) of tile t,
    // rounded to bf16, with both row sums: added to l_f / l_b directly, or
    // (kSumCheck) first collected over the tile in tf / tb.
    bf16x8 pf[T::PS];
    float tf = 0.f, tb = 0.f;
    auto softmax = [&](int kb0, int kb1) {
#pragma unroll
      for (int kb = kb0; kb < kb1; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          f32x8 pv;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            pv[i] = fast_exp2(__builtin_fmaf(s_cur[kb][hf * 8 + i], p.scale_log2, -msub));
          pf[kb * 2 + hf] = to_bf16x8(pv);
          if constexpr (kSumCheck) {
            const bool first = kb == kb0 && hf == 0;
            tf = first ? sum_f32x8(pv) : tf + sum_f32x8(pv);
            tb = sum_bf16x8(pf[kb * 2 + hf], first ? 0.f : tb);
          } else {
            l_f += sum_f32x8(pv);
            l_b = sum_bf16x8(pf[kb * 2 + hf], l_b);
          }
        }
    };
    // fp8 Q K^T has half the matrix work of bf16: half of the softmax then runs
    // beside the P V products of block B instead.
    constexpr bool kSplit = FP8;
    constexpr int KB_A = kSplit ? T::KB / 2 : T::KB;

    // Block A. Its DMA of K(t+2) and V(t+1) has no branch: a step before the
    // last always has a next tile, and a K tile past the visited range is
    // issued over an empty range (zeros land in a free ring slot), so the
    // loads can be scheduled among the matrix-core products.
    if constexpr (!LAST) {
      qk(kslot_next, s_nxt);
      ring_fence_before_copy();
      issue_k(t + 2 < ntiles ? kt + 2 : Nk / BN + 1, KRING + (1 - kslot_next) * T::KTILE);
      issue(vbase, kt + 1, VRING + (1 - vslot) * T::TILE);
      ring_fence_after_copy();
    }
    softmax(0, KB_A);
    // d = 64: explicit interleaving of the two blocks, with the boundary mask
    // between them so that each block is one straight-line region (measured
    // ~7 % faster at d = 64). At d = 128 the compiler's own order of block A
    // is faster, and block B is software-pipelined below.
    constexpr bool kInterleave = (D == 64) && !FP8;
    if constexpr (kInterleave && !LAST) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < T::KB * T::KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // matrix op
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // vector ops
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      }
    }
    // s_nxt is read by the vector ALU below (mask, row max). With the tile-sum
    // test (d = 128) its first vector read comes after the P V products.
    if constexpr (!LAST && (!kSumCheck || kInterleave || kSerialRings)) mfma_drain();
    if constexpr (kSumCheck) {
      // A lane whose share of the tile's row sum exceeds the limit holds a P
      // above it (or an overflow): move the reference maximum of those rows
      // above this tile's maximum and redo the tile's softmax (rare).
      const bool over = !(tf <= kSumLimit);
      if (wave_any(over)) {
        // Both halves of a row must move together. The exchange runs in every
        // lane (under a short-circuit it would run only where `over` is false).
        const float ov = over ? 1.f : 0.f;
        const bool row_over = ov + swap_halves(ov) != 0.f;
        const float mx = row_max(s_cur);
        mfma_drain();  // O was last written by matrix-core instructions
        const float m_new = fmaxf(m_ref, mx);
        const float m_up = m_new + p.head_raw;
        const float m_set = __builtin_isfinite(m_up) ? m_up : m_new;
        const float alpha = row_over ? fast_exp2((m_ref - m_set) * p.scale_log2) : 1.f;
        if (row_over) m_ref = m_set;
        l_b *= alpha;
        l_f *= alpha;
#pragma unroll
        for (int i = 0; i < T::DB; ++i) oacc[i] *= alpha;
        msub = (m_ref == -kInf) ? 0.f : m_ref * p.scale_log2;
        softmax(0, T::KB);
      }
      l_f += tf;
      l_b += tb;
    }
    if (!LAST && kInterleave && mask_next) {
      if (COUNT) ++masked;
      mask_tile(kt + 1, s_nxt);
    }

    // Block B: O^T += V^T P^T. Two waves of different work-groups share each
    // SIMD; while this wave issues its matrix-core products it takes issue
    // priority, so the matrix core is fed while the other wave runs its
    // vector work (measured 3 % faster than equal priority).
    __builtin_amdgcn_s_setprio(2);
    const lds_u8* vt_lds = L + VRING + vslot * T::TILE;
    auto vread = [&](int db, int tt) -> bf16x8 {
      const uint2 lo = lds_tr_b64(vt_lds, voff[db][0] + tt * 16 * T::ROWB);
      const uint2 hi = lds_tr_b64(vt_lds, voff[db][1] + tt * 16 * T::ROWB);
      return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    if constexpr (kInterleave) {
#pragma unroll
      for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int tt = 0; tt < T::PS; ++tt) oacc[db] = mfma32x32x16(vread(db, tt), pf[tt], oacc[db]);
    } else {
      // Software-pipelined by key step: the V^T operands of step tt + 1 are
      // read while the DB independent products of step tt issue, so no
      // product waits for its own LDS read.
      bf16x8 va[2][T::DB];
#pragma unroll
      for (int db = 0; db < T::DB; ++db) va[0][db] = vread(db, 0);
#pragma unroll
      for (int tt = 0; tt < T::PS; ++tt) {
        if (kSplit && tt == 2 * KB_A) softmax(KB_A, T::KB);
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          oacc[db] = mfma32x32x16(va[tt & 1][db], pf[tt], oacc[db]);
          if (tt + 1 < T::PS) va[(tt + 1) & 1][db] = vread(db, tt + 1);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * T::DB, 2);
#pragma unroll
      for (int i = 0; i < T::DB * T::PS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
        if (i < T::DB * (T::PS - 1)) __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
      }
    }
    if constexpr (LAST) {
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    if (!kInterleave && mask_next) {
      if (COUNT) ++masked;
      mask_tile(kt + 1, s_nxt);
    }
    const float mx = kSumCheck ? 0.f : row_max(s_nxt);
    if constexpr (kInterleave) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
      for (int i = 0; i < T::DB * T::PS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    wait_vmem();
    __syncthreads();
    if constexpr (kSumCheck) {
      // Rows that have seen no key yet take their reference from the next
      // tile's maximum before its softmax (window and empty-row cases).
      if (wave_any(m_ref == -kInf)) rescale(row_max(s_nxt));
    } else {
      rescale(mx);
    }
  };

  f32x16 sA[T::KB], sB[T::KB];
  if (ntiles > 0) {
    issue_k(kt_lo, KRING);
    issue(vbase, kt_lo, VRING);
    if (COUNT) ++loaded;
    if (ntiles > 1) {
      issue_k(kt_lo + 1, KRING + T::KTILE);
      if (COUNT) ++loaded;
    }
    wait_vmem();
    __syncthreads();
    qk(0, sA);
    mfma_drain();
    if (tile_partial(kt_lo)) {
      if (COUNT) ++masked;
      mask_tile(kt_lo, sA);
    }
    rescale(row_max(sA));
    __syncthreads();  // K slot 0 is refilled by the first step
  }
  using Mid = std::false_type;
  using Last = std::true_type;
  int t = 0;
  for (; t + 2 < ntiles; t += 2) {
    step(Mid{}, t, 1, 0, sA, sB, tile_partial(kt_lo + t + 1));
    step(Mid{}, t + 1, 0, 1, sB, sA, tile_partial(kt_lo + t + 2));
  }
  if (t + 2 == ntiles) {
    step(Mid{}, t, 1, 0, sA, sB, tile_partial(kt_lo + t + 1));
    step(Last{}, t + 1, 0, 1, sB, sA, false);
  } else if (t + 1 == ntiles) {
    step(Last{}, t, 1, 0, sA, sB, false);
  }
  mfma_drain();

  // Epilogue: O = acc / l, LSE = m * scale + ln l.
  const float lb = l_b + swap_halves(l_b);
  const float lf = l_f + swap_halves(l_f);
  const float inv = lb > 0.f ? 1.f / lb : 0.f;
  // This lane's row, recomputed from the lane counter rather than kept live
  // across the key loop (the loop has no register to spare for it).
  const int lane_e = lane_id();
  const int ge = lane_e >> 5;
  const int qrow_e = q0 + wave * 32 + (lane_e & 31);
  // O goes to device memory through LDS (store_rows_bf16), each wave's 32
  // rows in its own 64 D bytes from offset 0. With bf16 K that is the K ring,
  // which no wave reads after the last step's barrier (and whose copies that
  // barrier has seen land); the fp8 K ring is smaller, so there the
  // work-group first waits for every wave.
  if constexpr (FP8) __syncthreads();
  {
    uint2 w[D / 8];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        w[db * 4 + rr].x = pack_bf16x2(oacc[db][rr * 4 + 0] * inv, oacc[db][rr * 4 + 1] * inv);
        w[db * 4 + rr].y = pack_bf16x2(oacc[db][rr * 4 + 2] * inv, oacc[db][rr * 4 + 3] * inv);
      }
    const int row0 = q0 + wave * 32;
    store_rows_bf16<D>(L + wave * 64 * D, w, lane_e, p.o + (head_q + row0) * D, Nq - row0);
  }
  if (qrow_e < Nq && ge == 0 && p.lse != nullptr)
    p.lse[head_q + qrow_e] = lf > 0.f ? m_ref * p.scale + fast_log2(lf) * kLn2 : -kInf;
  if (COUNT && tid == 0) {
    int* c = p.counts + 2 * ((size_t)(b * p.H + h) * p.nqt + qt);
    c[0] = loaded;
    c[1] = masked;
  }
}

template <int D>
hipError_t launch_d(const FwdParams& prm, hipStream_t stream, bool count, bool fp8) {
  const unsigned nblk = (unsigned)((size_t)prm.B * prm.H * prm.nqt);
  void* args[] = {const_cast<FwdParams*>(&prm)};
  const bool c0 = prm.causal && prm.window == 0;
  const void* fn = fp8 ? (c0 ? reinterpret_cast<const void*>(&fwd_bf16_kernel<D, false, true, true>)
                             : reinterpret_cast<const void*>(&fwd_bf16_kernel<D, false, true>))
                   : count ? reinterpret_cast<const void*>(&fwd_bf16_kernel<D, true>)
                   : c0    ? reinterpret_cast<const void*>(&fwd_bf16_kernel<D, false, false, true>)
                           : reinterpret_cast<const void*>(&fwd_bf16_kernel<D, false>);
  return hipLaunchKernel(fn, dim3(nblk), dim3(kThreads), args, 0, stream);
}

}  // namespace

void fwd_bf16_tile_shape(int d, int* block_m, int* block_n) {
  *block_m = kBM;
  *block_n = d == 128 ? Tile<128>::BN : Tile<64>::BN;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.B = a.B;
  p.H = a.H;
  p.Hkv = a.Hkv;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.G = a.H / a.Hkv;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  p.thr_raw = kRescaleThreshold / p.scale_log2;
  p.head_raw = kRescaleHeadroom / p.scale_log2;
  if (!std::isfinite(p.head_raw)) p.head_raw = 0.f;
  p.causal = a.causal;
  p.window = a.window;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.nqt = ((a.cu_q != nullptr ? a.max_q : a.Nq) + kBM - 1) / kBM;
  p.xcd_remap = ((a.B * a.Hkv) % 8 == 0) ? 1 : 0;
  p.counts = a.counts;
  if (log_enabled())
    fprintf(stderr, "[miattn] fwd_bf16 d=%d grid=%lld block=%d BM=%d BN=%d xcd_remap=%d\n", a.d,
            (long long)a.B * a.H * p.nqt, kThreads, kBM, Tile<128>::BN, p.xcd_remap);
  const bool count = a.counts != nullptr;
  return a.d == 128 ? launch_d<128>(p, stream, count, a.fp8 != 0)
                    : launch_d<64>(p, stream, count, a.fp8 != 0);
}

}  // namespace miattn
