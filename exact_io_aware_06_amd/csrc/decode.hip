// Split-K decode (one query token per sequence against a KV cache) and the
// log-sum-exp merge of its partial results, gfx950.
//
// Decode is bound by reading the KV cache once per step ("Attention
// Research", section 1; "Quadratic Complexity Bottleneck", KV cache entry).
// Split-K over keys ("Attention Research", section 2) gives the GPU enough
// independent work. With equal lengths, each sequence's Nk cache rows are cut
// into S contiguous chunks, and each (sequence, KV head, chunk) becomes one
// work-group that reads its K/V rows exactly once for all G query heads
// sharing that KV head. With per-sequence lengths, a plan lays the visible
// keys of all sequences end to end in tiles (computed by every split
// work-group itself for up to 256 sequences, by a small plan kernel for
// larger batches), and each of the
// work-groups per KV head (at most B * S, and at most one round of the
// work-groups the device holds at once) takes an equal run of whole tiles
// (each sequence counted one tile longer, for what a piece costs beyond its
// tiles), cut at sequence boundaries into pieces (one partial each), so a
// long sequence in a batch of short ones is spread over the machine instead
// of over S chunks.
//
// A paged cache changes only where a key row is read from: row j of a
// sequence lives in page block_table[b][j / page_size] of a page pool, at row
// j % page_size ("Attention Research", section 2, names paged variants of the
// attention kernels).
//
// Split kernel: the work-group walks its chunk in tiles of 128 keys staged
// through LDS. Every thread loads whole 16-byte pieces of four consecutive K
// and V rows with non-temporal loads (the cache is streamed once; with
// row-contiguous accesses this runs ~7 % faster than cached loads), and
// stores them as rows: K padded, V XOR-swizzled, read back as V^T with
// transposing LDS reads as in the prefill kernel. Wave w
// takes keys [32w, 32w + 32) of each tile and treats the G query heads as the
// 32 columns of a transposed score tile S^T = K Q^T (columns >= G are zero
// and discarded); a group of more than 32 query heads is split into blocks of
// 32, one work-group each, which read the same keys. Each wave keeps its own
// running max / sum / output; at the end the four waves are combined through
// LDS into one normalised partial O_s and its lse_s = ln sum exp(scores) for
// the chunk (a work-group whose run of tiles spans several sequences does
// this once per piece).
//
// Merge kernel: per (sequence, query head), LSE = ln sum_s exp(lse_s) and
// O = sum_s exp(lse_s - LSE) O_s; chunks with no visible key have
// lse_s = -inf and weigh nothing.

#include <algorithm>
#include <cstdio>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace miattn {

// Scratch memory of the no-allocation decode entry point: the split partials
// live here instead of in a caller workspace. Every GPU that runs the library
// holds its own copy for the life of the process. The host never uses this
// name as an address (on the host it is only a handle of the symbol); the
// device address of the current GPU's copy comes from decode_scratch().
__device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
// Work-groups of the balanced split kernel (d = 128, d = 64) resident on a
// device at once (compute units x work-groups per compute unit); 0 = not yet
// queried.
std::mutex g_slots_mu;
int g_slots[kMaxDevices][2] = {};
}  // namespace

hipError_t decode_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    // The caller has made `device` current: this resolves that device's copy.
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 128;  // keys per tile: four waves x 32
// Balanced pieces: the plan counts each sequence that has keys as this many
// tiles more than it holds (virtual tiles, at the start of its run), for
// what a piece costs beyond its tiles (Q reload, the first tile's load
// latency, the combine), so that a work-group whose run crosses many short
// sequences gets fewer real tiles. Same-process A/B, one against none: a batch of
// 8 x 32768 and 56 x 512 keys 0.1956 -> 0.1900 ms, 64 random lengths in
// [1, 2047] 0.0543 -> 0.0528 ms, equal and uniform-random lengths unchanged;
// two virtual tiles gained less.
constexpr int kPieceUnits = 1;
// Batches of at most this many sequences (one per thread of a work-group) have
// their plan computed by every split work-group itself, without the plan
// kernel and its launch (same-process A/B, bit-identical: the skewed batch
// 0.1906 -> 0.1869 ms, 64 random lengths in [1, 2047] 0.0528 -> 0.0495 ms,
// the uniform random lengths of 32768-key slots 0.6606 -> 0.6572 ms).
constexpr int kFoldMaxB = 256;
constexpr float kRescaleThreshold = 8.0f;

struct SplitParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o_s;
  float* lse_s;
  int B, H, Hkv, Nk, G, S;
  int HB;  // blocks of up to 32 query heads per K/V head (ceil(G / 32))
  int window;
  float scale, scale_log2, thr_raw;
  const int* kv_lens;  // per-sequence key counts, or null (all Nk)
  // Balanced pieces (per-sequence lengths): the plan, tcum[0..B] = running
  // sum of the sequences' units (visible tiles plus kPieceUnits), tcum[B + 1]
  // = units per work-group, tcum[B + 2 + w] = the sequence holding
  // work-group w's first unit. decode_plan_kernel writes it and the split
  // kernel reads it, or (FOLD, B <= kFoldMaxB) every split work-group
  // computes tcum[0..B + 1] itself, for W work-groups per unit, and
  // work-group 0 writes that much of it here for the merge.
  int* tcum;
  int W;
  // Paged cache: k, v are page pools [num_pages, Hkv, page_size, d] and
  // block_table [B, max_pages] names the physical page of each sequence's
  // j-th run of page_size keys (Nk = max_pages * page_size).
  const int* block_table;
  int page_shift;  // log2(page_size)
  int max_pages, num_pages;
};

struct MergeParams {
  const float* o_s;
  const float* lse_s;
  uint16_t* o;
  float* lse;
  int BH, S, H;
  const int* tcum;  // balanced pieces: the plan (see SplitParams), else null
};

struct PlanParams {
  const int* kv_lens;
  int* tcum;
  int B, Nk, window;
  int W;  // work-groups of the split grid per (KV head, head block)
};

template <int D>
struct DTile {
  static constexpr int KSTR = D + 8;
  static constexpr int STAGE = kBN * KSTR + kBN * D;  // K rows (padded), V rows (swizzled)
  static constexpr int DB = D / 32;
  static constexpr int KS = D / 16;
  static constexpr int DCH = D / 8;
  static constexpr int KCH = kBN / 4;
  static constexpr int NB = KCH * DCH / kThreads;  // 4x8 blocks per thread per tile
  static_assert(NB * kThreads == KCH * DCH, "tile blocks must split evenly");
  static constexpr int VROWB = D * 2;  // bytes per V row in LDS
  // The end-of-chunk combine reuses the tile storage.
  static_assert((4 * 32 * D + 3 * 4 * 32) * 4 <= STAGE * 2, "combine scratch fits");
};

// V tile in LDS: row-major [key][d] with the 16-byte chunks of each row
// XOR-swizzled (as in the prefill kernel), so that rows are stored with
// plain 16-byte writes and the transposing V^T operand reads are free of bank
// conflicts.
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const uint16_t* p, bool ok) {
  if (!ok) return make_uint4(0u, 0u, 0u, 0u);
  const u32x4_nt x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

template <int D>
__device__ __forceinline__ int vswz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D, bool PAGED, bool BAL, bool FOLD = false>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(SplitParams p) {
  using T = DTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[T::STAGE];
  // Paged cache: the page id of every row of the next tile to load, in two
  // slots. Row r of tile t (starting at t0) reads slot t % 2, entry r - t0.
  __shared__ int pid[PAGED ? 2 : 1][PAGED ? kBN : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  // The work of this work-group: (KV head, head block), and either
  //  * equal chunks (!BAL): chunk s of sequence b, keys [s C, s C + C) with
  //    C = ceil(n / S), or
  //  * balanced pieces (BAL): the work-group's share [g_lo, g_hi) of the
  //    batch's units laid end to end (sequence b owns units [tcum[b],
  //    tcum[b + 1]) of that list: kPieceUnits virtual ones, then its visible
  //    key tiles from its first visible key), cut at sequence boundaries into
  //    pieces; the piece of (work-group w, sequence b) is partial w + b among
  //    each query head's B (S + 1) rows.
  // Grid order: split (work-group share) slowest. Consecutive work-groups are
  // different units of the same split, so the XCDs, which receive
  // work-groups round-robin, each get the same mix of work.
  const int nunit = BAL ? p.Hkv * p.HB : p.B * p.Hkv * p.HB;
  const int s = blockIdx.x / nunit;
  const int unit = blockIdx.x - s * nunit;
  const int hb = unit % p.HB;
  const int bk = unit / p.HB;
  const int g0 = hb * 32;               // first query head of this block in the group
  const int GB = min(32, p.G - g0);     // query heads in this block
  const int kvh = bk % p.Hkv;

  int b, start, hi, ntiles, g_lo = 0, g_hi = 0;
  // Sequence b's keys: its first n cache rows (the query sits at n - 1); the
  // window keeps the last W + 1.
  auto seq_keys = [&](int bb, int& vis) -> int {
    const int n = p.kv_lens != nullptr ? min(max(p.kv_lens[bb], 0), p.Nk) : p.Nk;
    vis = p.window > 0 ? max(0, n - 1 - p.window) : 0;
    return n;
  };
  // Balanced pieces, folded plan: the running unit counts in LDS.
  __shared__ int tc_lds[FOLD ? kFoldMaxB + 1 : 1];
  __shared__ int fold_tmp[FOLD ? kThreads / 64 + 1 : 1];
  // (LDS values are the same in every lane: readfirstlane keeps them, and the
  // branches on them, scalar.)
  auto cum = [&](int i) -> int {
    if constexpr (FOLD) return __builtin_amdgcn_readfirstlane(tc_lds[i]);
    return p.tcum[i];
  };
  // BAL: the piece of sequence b inside [g_lo, g_hi).
  auto piece = [&]() {
    int vis;
    const int n = seq_keys(b, vis);
    const int tb = cum(b), tb1 = cum(b + 1);
    // This share's units of the sequence, less its virtual tiles (a share
    // that holds only those gets an empty piece, whose partial weighs nothing).
    const int t_lo = max(0, max(tb, g_lo) - tb - kPieceUnits);
    const int t_hi = max(0, min(tb1, g_hi) - tb - kPieceUnits);
    start = vis + t_lo * kBN;
    hi = min(n, vis + t_hi * kBN);
    ntiles = t_hi - t_lo;
  };
  if constexpr (BAL) {
    int total, budget;
    if constexpr (FOLD) {
      // The plan of decode_plan_kernel, for B <= kThreads: thread b holds
      // sequence b's units; an inclusive scan over the work-group gives the
      // running counts.
      int t = 0;
      if (tid < p.B) {
        int vis;
        const int n = seq_keys(tid, vis);
        t = (n - vis + kBN - 1) / kBN;
        t = t > 0 ? t + kPieceUnits : 0;
      }
      int x = t;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (lane == 63) fold_tmp[wave] = x;
      __syncthreads();
      int before = 0;
      total = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) {
        before += w < wave ? fold_tmp[w] : 0;
        total += fold_tmp[w];
      }
      total = __builtin_amdgcn_readfirstlane(total);
      if (tid < p.B) tc_lds[tid + 1] = before + x;
      if (tid == 0) tc_lds[0] = 0;
      budget = max(1, (total + p.W - 1) / p.W);
      __syncthreads();
      // The merge reads the running counts and the budget; work-group 0
      // publishes them (also when every sequence is empty).
      if (blockIdx.x == 0) {
        for (int i = tid; i <= p.B; i += kThreads) p.tcum[i] = tc_lds[i];
        if (tid == 0) p.tcum[p.B + 1] = budget;
      }
      g_lo = s * budget;
      if (g_lo >= total) return;  // the batch's units are all taken by earlier work-groups
      // The sequence that owns unit g_lo (exactly one, since g_lo < total).
      if (tid < p.B && tc_lds[tid] <= g_lo && g_lo < tc_lds[tid + 1]) fold_tmp[kThreads / 64] = tid;
      __syncthreads();
      b = __builtin_amdgcn_readfirstlane(fold_tmp[kThreads / 64]);
    } else {
      total = p.tcum[p.B];
      budget = p.tcum[p.B + 1];
      g_lo = s * budget;
      if (g_lo >= total) return;  // the batch's units are all taken by earlier work-groups
      b = p.tcum[p.B + 2 + s];    // the sequence that owns unit g_lo
    }
    g_hi = min(total, g_lo + budget);
    piece();
  } else {
    b = bk / p.Hkv;
    int vis;
    const int n = seq_keys(b, vis);
    const int C = (n + p.S - 1) / p.S;
    const int lo = min(n, s * C);
    hi = min(n, lo + C);
    start = max(lo, vis);
    ntiles = hi > start ? (hi - start + kBN - 1) / kBN : 0;
  }

  // Query heads of this group as the B-operand columns.
  const bool qvalid = l32 < GB;
  const int hq = kvh * p.G + g0 + (qvalid ? l32 : 0);
  bf16x8 qf[T::KS];
  auto load_q = [&]() {
    const uint16_t* qp = p.q + ((size_t)b * p.H + hq) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) qf[ks] = as_bf16x8(load16(qp + ks * 16, qvalid));
  };
  load_q();

  const int page_mask = (1 << p.page_shift) - 1;
  // Paged: thread tid < kBN reads the block-table entry of row t0 + tid (one
  // iteration before the rows themselves are loaded, so the table read is off
  // the load's critical path); rows past the chunk get -1.
  auto fetch_pid = [&](int t0) -> int {
    const int r = t0 + tid;
    return (tid < kBN && r < hi) ? p.block_table[(size_t)b * p.max_pages + (r >> p.page_shift)]
                                 : -1;
  };
  // Element offset of cache row r (< hi) of tile t0 in page-id slot `slot`,
  // and whether it may be read: a page id outside the pool reads as zeros.
  auto row_at = [&](int r, int t0, int slot, bool& ok) -> size_t {
    if (!PAGED) return (((size_t)b * p.Hkv + kvh) * p.Nk + (size_t)r) * D;
    const int pg = pid[slot][r - t0];
    ok = ok && (unsigned)pg < (unsigned)p.num_pages;
    const size_t page = ok ? (size_t)pg : 0;
    return (((page * p.Hkv + kvh) << p.page_shift) + (size_t)(r & page_mask)) * D;
  };

  uint4 kreg[T::NB][4], vreg[T::NB][4];
  // V^T operand of the products below, by transposing reads: as a source lane
  // of its 16-lane group this lane names rows 4g + e (+8 for the second read)
  // of a 16-key step and dims db*32 + 16hh + 4a'; lane 16hh + i then receives
  // dims 16hh + i of keys 4g..4g+3 and 8+4g..8+4g+3 of the step, the key order
  // of this lane's P registers.
  uint32_t voff[T::DB][2];
  {
    const int j = lane & 15, a = j & 3, e = j >> 2, hh = (lane >> 4) & 1;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int r = 4 * g + e + 8 * qh;
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const int c = 4 * db + 2 * hh + (a >> 1);
        voff[db][qh] = (uint32_t)(r * T::VROWB + ((c ^ vswz<D>(r)) << 4) + (a & 1) * 8);
      }
    }
  }
  auto load_tile = [&](int t0, int slot) {
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb) {
      const int bi = tid + nb * kThreads;
      const int kc = bi / T::DCH, dc = bi % T::DCH;  // rows 4 kc .. + 3, chunk dc
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rk = t0 + kc * 4 + r;
        bool ok = rk < hi;
        const size_t off = row_at(ok ? rk : t0, t0, slot, ok);
        kreg[nb][r] = load16_nt(p.k + off + dc * 8, ok);
        vreg[nb][r] = load16_nt(p.v + off + dc * 8, ok);
      }
    }
  };
  auto store_tile = [&]() {
    uint16_t* ks = smem;
    uint16_t* vs = smem + kBN * T::KSTR;
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb) {
      const int bi = tid + nb * kThreads;
      const int kc = bi / T::DCH, dc = bi % T::DCH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = kc * 4 + r;
        *reinterpret_cast<uint4*>(ks + row * T::KSTR + dc * 8) = kreg[nb][r];
        *reinterpret_cast<uint4*>(vs + row * D + ((dc ^ vswz<D>(row)) * 8)) = vreg[nb][r];
      }
    }
  };

  // Partial-result row of query head g0 + col of this chunk or piece.
  auto prow = [&](int col) -> size_t {
    const int h = kvh * p.G + g0 + col;
    // Balanced pieces: head-major, so that one sequence's pieces are adjacent rows.
    return BAL ? (size_t)h * ((size_t)p.B * (p.S + 1)) + s + b : ((size_t)b * p.H + h) * p.S + s;
  };

  for (;;) {
    f32x16 oacc[T::DB];
#pragma unroll
    for (int i = 0; i < T::DB; ++i) oacc[i] = f32x16{};
    float m_ref = -kInf;
    float l_b = 0.f, l_f = 0.f;  // row sums of the bf16-rounded and the fp32 P

    int pid_next = -1;  // paged: page id of this thread's row of the tile after the next
    if (ntiles > 0) {
      if (PAGED) {
        if (tid < kBN) pid[0][tid] = fetch_pid(start);
        if (ntiles > 1) pid_next = fetch_pid(start + kBN);
        __syncthreads();
      }
      load_tile(start, 0);
    }
    for (int it = 0; it < ntiles; ++it) {
      const int t0 = start + it * kBN;
      __syncthreads();  // every wave is done with the previous tile
      store_tile();
      if (PAGED && tid < kBN) pid[(it + 1) & 1][tid] = pid_next;  // rows of tile it + 1
      __syncthreads();
      if (it + 1 < ntiles) {
        load_tile(t0 + kBN, (it + 1) & 1);
        if (PAGED && it + 2 < ntiles) pid_next = fetch_pid(t0 + 2 * kBN);
      }

      const uint16_t* ks = smem;
      const uint16_t* vs = smem + kBN * T::KSTR;
      f32x16 sacc = f32x16{};
      {
        const uint16_t* kp = ks + (wave * 32 + l32) * T::KSTR + g * 8;
#pragma unroll
        for (int st = 0; st < T::KS; ++st)
          sacc = mfma32x32x16(lds_read_bf16x8(kp + st * 16), qf[st], sacc);
      }
      mfma_drain();
      if (t0 + kBN > hi) {
        const int lim = hi - (t0 + wave * 32 + 4 * g);  // offsets >= lim are past the chunk
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + (r & 3);
          sacc[r] = c < lim ? sacc[r] : -kInf;
        }
      }
      float mx = -kInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_ref, mx);
      const bool need = m_new > m_ref + p.thr_raw;
      if (wave_any(need)) {
        const float alpha = need ? fast_exp2((m_ref - m_new) * p.scale_log2) : 1.f;
        if (need) m_ref = m_new;
        l_b *= alpha;
        l_f *= alpha;
#pragma unroll
        for (int i = 0; i < T::DB; ++i) oacc[i] *= alpha;
      }
      const float msub = (m_ref == -kInf) ? 0.f : m_ref * p.scale_log2;
      bf16x8 pf[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x8 pv;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pv[i] = fast_exp2(__builtin_fmaf(sacc[hf * 8 + i], p.scale_log2, -msub));
        l_f += sum_f32x8(pv);
        pf[hf] = to_bf16x8(pv);
        l_b = sum_bf16x8(pf[hf], l_b);
      }
      const lds_u8* vl = lds_ptr((void*)vs) + wave * 32 * T::VROWB;  // this wave's 32 keys
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          const uint2 lo = lds_tr_b64(vl, voff[db][0] + t * 16 * T::VROWB);
          const uint2 hi2 = lds_tr_b64(vl, voff[db][1] + t * 16 * T::VROWB);
          const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi2.x, hi2.y));
          oacc[db] = mfma32x32x16(va, pf[t], oacc[db]);
        }
      mfma_drain();
    }

    // Combine the four waves' (max, sum, un-normalised output) per head.
    const float lb_col = l_b + swap_halves(l_b);
    const float lf_col = l_f + swap_halves(l_f);
    __syncthreads();  // tile storage is free again
    float* ow = reinterpret_cast<float*>(smem);   // [4][32][D]
    float* mw = ow + 4 * 32 * D;                  // [4][32]
    float* lbw = mw + 4 * 32;                     // [4][32] sums of rounded P
    float* lfw = lbw + 4 * 32;                    // [4][32] sums of fp32 P
    if (qvalid) {
      float* dst = ow + (wave * 32 + l32) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<f32x4*>(dst + db * 32 + rr * 8) =
              f32x4{oacc[db][rr * 4], oacc[db][rr * 4 + 1], oacc[db][rr * 4 + 2],
                    oacc[db][rr * 4 + 3]};
      if (g == 0) {
        mw[wave * 32 + l32] = m_ref;
        lbw[wave * 32 + l32] = lb_col;
        lfw[wave * 32 + l32] = lf_col;
      }
    }
    __syncthreads();
    for (int idx = tid; idx < GB * D; idx += kThreads) {
      const int col = idx / D, dim = idx - col * D;
      float M = -kInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, mw[w * 32 + col]);
      float Lb = 0.f, Lf = 0.f, acc = 0.f;
      if (M != -kInf) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float mwv = mw[w * 32 + col];
          const float e = mwv == -kInf ? 0.f : fast_exp2((mwv - M) * p.scale_log2);
          Lb += e * lbw[w * 32 + col];
          Lf += e * lfw[w * 32 + col];
          acc += e * ow[(w * 32 + col) * D + dim];
        }
      }
      const size_t row = prow(col);
      p.o_s[row * D + dim] = Lb > 0.f ? acc / Lb : 0.f;
      if (dim == 0) p.lse_s[row] = Lf > 0.f ? M * p.scale + fast_log2(Lf) * kLn2 : -kInf;
    }

    if constexpr (!BAL) {
      break;
    } else {
      if (cum(b + 1) >= g_hi) break;
      // The next sequence that owns units (one does: this share goes on).
      do {
        ++b;
      } while (cum(b + 1) == cum(b));
      piece();
      load_q();
    }
  }
}

// Plan of the balanced pieces (one work-group): sequence b owns
// t_b = ceil((n_b - vis_b) / kBN) tiles of the batch's visible keys, plus
// kPieceUnits virtual ones when t_b > 0; tcum is the running sum of those
// units, every work-group of the split grid takes ceil(total / W)
// consecutive units of that list, and for each work-group that gets any, the
// sequence holding its first unit is recorded.
__global__ __launch_bounds__(kThreads) void decode_plan_kernel(PlanParams p) {
  __shared__ int wsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < p.B; base += kThreads) {
    const int b = base + tid;
    int t = 0;
    if (b < p.B) {
      const int n = min(max(p.kv_lens[b], 0), p.Nk);
      const int vis = p.window > 0 ? max(0, n - 1 - p.window) : 0;
      t = (n - vis + kBN - 1) / kBN;
      t = t > 0 ? t + kPieceUnits : 0;
    }
    int x = t;  // inclusive running sum within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry, all = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      before += w < wave ? wsum[w] : 0;
      all += wsum[w];
    }
    if (b < p.B) p.tcum[b] = before + x - t;
    carry += all;
    __syncthreads();  // wsum is rewritten by the next round
  }
  const int total = carry;
  const int budget = max(1, (total + p.W - 1) / p.W);
  if (tid == 0) {
    p.tcum[p.B] = total;
    p.tcum[p.B + 1] = budget;
  }
  __syncthreads();  // every running sum is written
  for (int b = tid; b < p.B; b += kThreads) {
    const int tb = p.tcum[b], tb1 = b + 1 < p.B ? p.tcum[b + 1] : total;
    // Work-groups whose first tile w * budget lies in [tb, tb1).
    for (int w = (tb + budget - 1) / budget; w * budget < tb1; ++w) p.tcum[p.B + 2 + w] = b;
  }
}

template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(MergeParams p) {
  constexpr int DPL = D / 64;  // dims per lane
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  // This (sequence, head)'s partials: rows first .. first + count - 1.
  size_t first = (size_t)bh * p.S;
  int count = p.S;
  if (p.tcum != nullptr) {
    // Balanced pieces: work-groups w_lo .. w_hi hold sequence b's tiles, and
    // the piece of (w, b) is partial w + b of head h's B (S + 1) rows.
    const int b = bh / p.H, h = bh - b * p.H;
    const int tb = p.tcum[b], tb1 = p.tcum[b + 1], budget = p.tcum[p.BH / p.H + 1];
    const int w_lo = tb / budget;
    count = tb1 > tb ? (tb1 - 1) / budget - w_lo + 1 : 0;
    first = (size_t)h * ((size_t)(p.BH / p.H) * (p.S + 1)) + w_lo + b;  // head-major rows
  }
  const float* ls = p.lse_s;
  const float* os = p.o_s;
  float M = -kInf;
  for (int s = lane; s < count; s += 64) M = fmaxf(M, ls[first + s]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) M = fmaxf(M, __shfl_xor(M, w, 64));
  float L = 0.f, acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  if (M != -kInf) {
    for (int s = 0; s < count; ++s) {
      const size_t row = first + s;
      const float lv = ls[row];
      const float w = lv == -kInf ? 0.f : expf(lv - M);
      L += w;
#pragma unroll
      for (int i = 0; i < DPL; ++i)
        acc[i] = __builtin_fmaf(w, os[row * D + lane * DPL + i], acc[i]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* op = p.o + (size_t)bh * D + lane * DPL;
  if (DPL == 2) {
    *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(acc[0] * inv, acc[DPL - 1] * inv);
  } else {
    const uint32_t w = pack_bf16x2(acc[0] * inv, 0.f);
    *op = (uint16_t)(w & 0xffffu);
  }
  if (lane == 0 && p.lse != nullptr) p.lse[bh] = L > 0.f ? M + logf(L) : -kInf;
}

}  // namespace

// Partial rows: B * H * S for equal chunks; with balanced pieces, one per
// (work-group share w < B * S, sequence b) pair that can occur, indexed
// w + b < B * (S + 1), per query head. Then the plan: B + 2 + B * S ints.
// Resident work-groups of split-kernel instantiation `which` (launched with
// kThreads threads) on the current device, cached per device.
hipError_t resident_work_groups(int which, const void* fn, int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_slots_mu);
  int& v = g_slots[dev][which];
  if (v == 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0);
    if (e != hipSuccess) return e;
    v = max(1, cus * per_cu);
  }
  *out = v;
  return hipSuccess;
}

size_t decode_workspace_bytes(int B, int H, int d, int splits) {
  const size_t rows = (size_t)B * H * (splits + 1);
  return rows * (size_t)(d + 1) * sizeof(float) + ((size_t)B * (splits + 1) + 2) * sizeof(int);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  SplitParams sp;
  sp.q = static_cast<const uint16_t*>(a.q);
  sp.k = static_cast<const uint16_t*>(a.k);
  sp.v = static_cast<const uint16_t*>(a.v);
  const size_t rows = (size_t)a.B * a.H * (a.splits + 1);
  sp.o_s = static_cast<float*>(a.workspace);
  sp.lse_s = sp.o_s + rows * a.d;
  int* plan = reinterpret_cast<int*>(sp.lse_s + rows);
  // Per-sequence lengths (and paged caches, which always have them) use
  // balanced pieces; equal lengths keep one equal chunk per work-group.
  const bool bal = a.kv_lens != nullptr;
  sp.tcum = bal ? plan : nullptr;
  const bool fold = bal && a.B <= kFoldMaxB;
  sp.B = a.B;
  sp.H = a.H;
  sp.Hkv = a.Hkv;
  sp.Nk = a.Nk;
  sp.G = a.H / a.Hkv;
  sp.HB = (sp.G + 31) / 32;
  sp.S = a.splits;
  sp.window = a.window;
  sp.kv_lens = a.kv_lens;
  sp.block_table = a.block_table;
  sp.page_shift = 0;
  while (a.block_table != nullptr && (1 << sp.page_shift) < a.page_size) ++sp.page_shift;
  sp.max_pages = a.max_pages;
  sp.num_pages = a.num_pages;
  sp.scale = a.scale;
  sp.scale_log2 = a.scale * kLog2e;
  sp.thr_raw = kRescaleThreshold / sp.scale_log2;
  const bool paged = a.block_table != nullptr;
  const void* sfn;
  if (a.d == 128)
    sfn = paged ? (fold ? reinterpret_cast<const void*>(&decode_split_kernel<128, true, true, true>)
                        : reinterpret_cast<const void*>(&decode_split_kernel<128, true, true>))
          : bal ? (fold ? reinterpret_cast<const void*>(&decode_split_kernel<128, false, true, true>)
                        : reinterpret_cast<const void*>(&decode_split_kernel<128, false, true>))
                : reinterpret_cast<const void*>(&decode_split_kernel<128, false, false>);
  else
    sfn = paged ? (fold ? reinterpret_cast<const void*>(&decode_split_kernel<64, true, true, true>)
                        : reinterpret_cast<const void*>(&decode_split_kernel<64, true, true>))
          : bal ? (fold ? reinterpret_cast<const void*>(&decode_split_kernel<64, false, true, true>)
                        : reinterpret_cast<const void*>(&decode_split_kernel<64, false, true>))
                : reinterpret_cast<const void*>(&decode_split_kernel<64, false, false>);
  // Equal chunks: B * S work-groups per (KV head, head block). Balanced
  // pieces: at most B * S, and no more than one round of the work-groups the
  // device holds at once, so each takes one long equal run of tiles (fewer,
  // longer work-groups pay the plan reads and the combine less often, and no
  // work-group waits for a second round).
  const size_t units = (size_t)a.Hkv * sp.HB;
  size_t per_unit = (size_t)a.B * a.splits;
  hipError_t e;
  if (bal) {
    // Sized from the contiguous instantiation for both caches, so that a paged
    // cache and a contiguous one holding the same keys get the same pieces.
    const void* sized = a.d == 128
                            ? reinterpret_cast<const void*>(&decode_split_kernel<128, false, true>)
                            : reinterpret_cast<const void*>(&decode_split_kernel<64, false, true>);
    int slots = 0;
    e = resident_work_groups(a.d == 128 ? 0 : 1, sized, &slots);
    if (e != hipSuccess) return e;
    per_unit = std::min(per_unit, std::max<size_t>(1, (size_t)slots / units));
  }
  const unsigned nsplit_blk = (unsigned)(units * per_unit);
  if (log_enabled())
    fprintf(stderr,
            "[miattn] decode d=%d splits=%d kv_lens=%s page_size=%d split_grid=%u "
            "merge_grid=%d\n",
            a.d, a.splits, bal ? "per-sequence (balanced pieces)" : "uniform",
            a.block_table != nullptr ? a.page_size : 0, nsplit_blk, a.B * a.H);
  sp.W = (int)per_unit;
  if (bal && !fold) {
    PlanParams pp{a.kv_lens, plan, a.B, a.Nk, a.window, (int)per_unit};
    void* pargs[] = {&pp};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_plan_kernel), dim3(1),
                        dim3(kThreads), pargs, 0, stream);
    if (e != hipSuccess) return e;
  }
  void* sargs[] = {&sp};
  e = hipLaunchKernel(sfn, dim3(nsplit_blk), dim3(kThreads), sargs, 0, stream);
  if (e != hipSuccess) return e;

  MergeParams mp;
  mp.o_s = sp.o_s;
  mp.lse_s = sp.lse_s;
  mp.o = static_cast<uint16_t*>(a.o);
  mp.lse = a.lse;
  mp.BH = a.B * a.H;
  mp.S = a.splits;
  mp.H = a.H;
  mp.tcum = sp.tcum;
  void* margs[] = {&mp};
  const void* mfn = a.d == 128 ? reinterpret_cast<const void*>(&decode_merge_kernel<128>)
                               : reinterpret_cast<const void*>(&decode_merge_kernel<64>);
  return hipLaunchKernel(mfn, dim3((unsigned)mp.BH), dim3(64), margs, 0, stream);
}

}  // namespace miattn
