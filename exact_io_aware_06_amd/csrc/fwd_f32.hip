// Fused attention forward in fp32 throughout (no bf16 rounding anywhere).
//
// Same algorithm as the bf16 kernel (tiled K/V streamed through LDS, online
// softmax with a running maximum and sum per query row, one normalise at the
// end; "Chapter 3.1 - The Cost of Attention", section 5), on the vector ALUs
// in fp32. It serves small, precision-critical shapes; it is not the
// throughput path.
//
// Each query row is owned by D / 32 consecutive lanes, each holding 32 of its
// dimensions of q and of the output accumulator; a dot product is a 32-term
// in-lane sum plus a butterfly over those lanes. The eight waves of a
// work-group hold the same query rows and split the key tiles between them
// (wave w takes tiles w, w + 8, ...), each staging its tiles in its own LDS
// region with 16-byte loads; their (max, sum, output) partials are merged
// once at the end, as the online softmax merges any two partial results.

#include <cstdio>

#include "common.hpp"
#include "launch.hpp"

namespace miattn {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, H, Hkv, Nq, Nk, G;
  float scale;
  int causal, window;
  int nqt;
};

template <int D>
struct F32Tile {
  static constexpr int TPQ = D / 32;     // lanes per query row
  static constexpr int BM = 64 / TPQ;    // query rows per work-group (one wave's worth)
  static constexpr int BN = 2048 / D;    // keys per wave tile (16 KB of K and V per wave)
};

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Params p) {
  using T = F32Tile<D>;
  constexpr int TPQ = T::TPQ, BM = T::BM, BN = T::BN;
  // per wave: K tile [BN][D] then V tile [BN][D]; reused for the final merge
  __shared__ __attribute__((aligned(16))) float lds[kWaves][2 * BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane % TPQ;
  const int bh = blockIdx.x / p.nqt;
  const int qt = p.nqt - 1 - (blockIdx.x - bh * p.nqt);
  const int b = bh / p.H, h = bh - b * p.H;
  const int kvh = h / p.G;
  const int q0 = qt * BM;
  const int qrow = q0 + lane / TPQ;
  const bool qvalid = qrow < p.Nq;
  const int off = p.Nk - p.Nq;
  const long long qpos = (long long)qrow + off;
  const int q_last = min(q0 + BM, p.Nq) - 1;
  const long long p_lo = (long long)q0 + off, p_hi = (long long)q_last + off;

  long long key_lo = 0, key_hi = p.Nk;
  if (p.causal) key_hi = min(key_hi, p_hi + 1);
  else if (p.window > 0) key_hi = min(key_hi, p_hi + p.window + 1);
  if (p.window > 0) key_lo = max(key_lo, p_lo - p.window);

  const size_t head_q = (size_t)(b * p.H + h) * p.Nq;
  const size_t head_kv = (size_t)(b * p.Hkv + kvh) * p.Nk;

  float qv[32], acc[32];
  for (int c = 0; c < 32; ++c) {
    qv[c] = qvalid ? p.q[(head_q + qrow) * D + sub * 32 + c] : 0.f;
    acc[c] = 0.f;
  }
  float m = -kInf, l = 0.f;
  float* ks = lds[wave];
  float* vs = lds[wave] + BN * D;

  if (key_hi > key_lo) {
    const int kt_lo = (int)(key_lo / BN), kt_hi = (int)((key_hi + BN - 1) / BN);
    for (int kt = kt_lo + wave; kt < kt_hi; kt += kWaves) {
      const int k0 = kt * BN;
      // this wave's lanes finished reading the previous tile (in-order LDS)
      __builtin_amdgcn_wave_barrier();
      // the tile's rows are contiguous in memory: 16-byte pieces, rows past
      // the keys read as zero
      const float4* kg = reinterpret_cast<const float4*>(p.k + (head_kv + k0) * D);
      const float4* vg = reinterpret_cast<const float4*>(p.v + (head_kv + k0) * D);
#pragma unroll
      for (int e4 = lane; e4 < BN * D / 4; e4 += 64) {
        const bool ok = k0 + (e4 * 4) / D < p.Nk;
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        reinterpret_cast<float4*>(ks)[e4] = ok ? kg[e4] : z;
        reinterpret_cast<float4*>(vs)[e4] = ok ? vg[e4] : z;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      float s[BN];
      float mx = -kInf;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c) dot = __builtin_fmaf(qv[c], ks[j * D + sub * 32 + c], dot);
#pragma unroll
        for (int w = 1; w < TPQ; w <<= 1) dot += __shfl_xor(dot, w, 64);
        const long long key = (long long)k0 + j;
        bool vis = key < p.Nk;
        if (p.causal) vis = vis && key <= qpos;
        if (p.window > 0) vis = vis && key >= qpos - p.window && (p.causal || key <= qpos + p.window);
        s[j] = vis ? dot * p.scale : -kInf;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m, mx);
      if (m_new == -kInf) continue;  // nothing visible to this row yet
      const float alpha = expf(m - m_new);  // m = -inf gives 0
      l *= alpha;
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] *= alpha;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        const float e = expf(s[j] - m_new);
        l += e;
#pragma unroll
        for (int c = 0; c < 32; ++c) acc[c] = __builtin_fmaf(e, vs[j * D + sub * 32 + c], acc[c]);
      }
      m = m_new;
    }
  }

  // Merge the waves' partials: each writes (m, l, acc) to its region,
  // then wave 0 combines them with weights exp(m_w - M).
  __syncthreads();
  {
    float* mine = lds[wave] + lane * 34;  // 34 floats per lane: m, l, 32 acc
    mine[0] = m;
    mine[1] = l;
    for (int c = 0; c < 32; ++c) mine[2 + c] = acc[c];
  }
  __syncthreads();
  if (wave == 0) {
    float M = -kInf;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds[w][lane * 34]);
    float L = 0.f, out[32];
    for (int c = 0; c < 32; ++c) out[c] = 0.f;
    if (M != -kInf) {
      for (int w = 0; w < kWaves; ++w) {
        const float* part = lds[w] + lane * 34;
        const float e = part[0] == -kInf ? 0.f : expf(part[0] - M);
        L += e * part[1];
        for (int c = 0; c < 32; ++c) out[c] = __builtin_fmaf(e, part[2 + c], out[c]);
      }
    }
    if (qvalid) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      for (int c = 0; c < 32; ++c) p.o[(head_q + qrow) * D + sub * 32 + c] = out[c] * inv;
      if (sub == 0 && p.lse != nullptr) p.lse[head_q + qrow] = L > 0.f ? M + logf(L) : -kInf;
    }
  }
}

}  // namespace

void fwd_f32_tile_shape(int d, int* block_m, int* block_n) {
  *block_m = 64 / (d / 32);
  *block_n = 2048 / d;
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  F32Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<float*>(a.o);
  p.lse = a.lse;
  p.B = a.B;
  p.H = a.H;
  p.Hkv = a.Hkv;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.G = a.H / a.Hkv;
  p.scale = a.scale;
  p.causal = a.causal;
  p.window = a.window;
  int bm, bn;
  fwd_f32_tile_shape(a.d, &bm, &bn);
  p.nqt = (a.Nq + bm - 1) / bm;
  const unsigned nblk = (unsigned)((size_t)a.B * a.H * p.nqt);
  if (log_enabled())
    fprintf(stderr, "[miattn] fwd_f32 d=%d grid=%u block=%d BM=%d BN=%d\n", a.d, nblk, kThreads,
            bm, bn);
  void* args[] = {&p};
  const void* fn = a.d == 128 ? reinterpret_cast<const void*>(&fwd_f32_kernel<128>)
                              : reinterpret_cast<const void*>(&fwd_f32_kernel<64>);
  return hipLaunchKernel(fn, dim3(nblk), dim3(kThreads), args, 0, stream);
}

}  // namespace miattn
