// libmiattn C ABI: argument validation, kernel selection, launch.
//
// Every argument is checked before the first HIP call so that argument errors
// are reported without touching (or needing) a device. No device memory is
// allocated here and nothing is synchronised.

#include <hip/hip_runtime_api.h>

#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>

#include "launch.hpp"
#include "miattn.h"

namespace miattn {

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("MIATTN_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

}  // namespace miattn

namespace {

using miattn::DecodeArgs;
using miattn::FwdArgs;

int device_status() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();  // do not leave a sticky error for the caller
    return MIATTN_ENODEVICE;
  }
  return MIATTN_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MIATTN_OK : MIATTN_ELAUNCH; }

bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

// Shared checks of the two forward entry points.
int check_fwd(const void* q, const void* k, const void* v, const void* o, int B, int H, int Hkv,
              int Nq, int Nk, int d, float scale, int causal, int window, int block_m) {
  if (B < 0 || H < 1 || Hkv < 1 || Nq < 0 || Nk < 0) return MIATTN_EINVAL;
  if (H % Hkv != 0) return MIATTN_EINVAL;
  if (causal != 0 && causal != 1) return MIATTN_EINVAL;
  if (window < 0) return MIATTN_EINVAL;
  if (!valid_scale(scale)) return MIATTN_EINVAL;
  if (d != 64 && d != 128) return MIATTN_EUNSUPPORTED;
  const long long nq_elems = (long long)B * H * Nq;
  const long long nk_elems = (long long)B * Hkv * Nk;
  if (nq_elems > 0 && (q == nullptr || o == nullptr)) return MIATTN_EINVAL;
  if (nq_elems > 0 && nk_elems > 0 && (k == nullptr || v == nullptr)) return MIATTN_EINVAL;
  // one work-group per (batch, head, query tile) in a 1-D grid
  const long long nqt = ((long long)Nq + block_m - 1) / block_m;
  if ((long long)B * H * nqt > (long long)INT_MAX) return MIATTN_EUNSUPPORTED;
  // K/V of one head are addressed through 32-bit buffer offsets
  if ((long long)Nk * d * 4 > 0xFFFFFFFFLL) return MIATTN_EUNSUPPORTED;
  return MIATTN_OK;
}

int run_fwd(bool f32, const void* q, const void* k, const void* v, void* o, float* lse, int B,
            int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
            int* counts, void* stream) {
  int bm = 0, bn = 0;
  if (d == 64 || d == 128) {
    if (f32) miattn::fwd_f32_tile_shape(d, &bm, &bn);
    else miattn::fwd_bf16_tile_shape(d, &bm, &bn);
  } else {
    bm = 1;
  }
  int st = check_fwd(q, k, v, o, B, H, Hkv, Nq, Nk, d, scale, causal, window, bm);
  if (st != MIATTN_OK) return st;
  if (B == 0 || Nq == 0) return MIATTN_OK;  // nothing to compute
  if ((st = device_status()) != MIATTN_OK) return st;
  FwdArgs a{q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, counts};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch_status(f32 ? miattn::launch_fwd_f32(a, s) : miattn::launch_fwd_bf16(a, s));
}

// Packed documents: same checks as check_fwd, on the packed sizes.
int run_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int* cu_q, const int* cu_k, int num_seqs, int H, int Hkv, int total_q,
                   int total_k, int max_q, int d, float scale, int causal, int window,
                   int* counts, void* stream) {
  if (num_seqs < 0 || H < 1 || Hkv < 1 || total_q < 0 || total_k < 0 || max_q < 0)
    return MIATTN_EINVAL;
  if (H % Hkv != 0) return MIATTN_EINVAL;
  if (causal != 0 && causal != 1) return MIATTN_EINVAL;
  if (window < 0 || !valid_scale(scale)) return MIATTN_EINVAL;
  if (d != 64 && d != 128) return MIATTN_EUNSUPPORTED;
  if (num_seqs > 0 && (cu_q == nullptr || cu_k == nullptr)) return MIATTN_EINVAL;
  if (total_q > 0 && (q == nullptr || o == nullptr)) return MIATTN_EINVAL;
  if (total_q > 0 && total_k > 0 && (k == nullptr || v == nullptr)) return MIATTN_EINVAL;
  int bm = 0, bn = 0;
  miattn::fwd_bf16_tile_shape(d, &bm, &bn);
  const long long nqt = ((long long)max_q + bm - 1) / bm;
  if ((long long)num_seqs * H * nqt > (long long)INT_MAX) return MIATTN_EUNSUPPORTED;
  if ((long long)total_k * d * 4 > 0xFFFFFFFFLL) return MIATTN_EUNSUPPORTED;
  if (num_seqs == 0 || max_q == 0 || total_q == 0) return MIATTN_OK;
  int st = device_status();
  if (st != MIATTN_OK) return st;
  FwdArgs a{q,     k,      v,      o,      lse,  num_seqs, H,    Hkv,  total_q,
            total_k, d, scale, causal, window, counts, cu_q,     cu_k, max_q};
  return launch_status(miattn::launch_fwd_bf16(a, static_cast<hipStream_t>(stream)));
}

int resolve_splits(int B, int Hkv, int Nk, int num_splits) {
  if (B < 0 || Hkv < 1 || Nk < 0 || num_splits < 0) return MIATTN_EINVAL;
  if (num_splits > 0) {
    if (Nk > 0 && num_splits > Nk) return MIATTN_EINVAL;
    if (Nk == 0 && num_splits > 1) return MIATTN_EINVAL;
    return num_splits;
  }
  // Library choice: about one round of the split kernel's resident
  // work-groups (256 compute units x 2), with chunks of at least 1024 keys.
  // Measured at H32 Hkv8 Nk32768 d128: B = 1, 4, 16, 64 take 32, 16, 4, 1
  // splits, each within 1 % of the fastest split count for its batch; the
  // earlier rule (about 2048 work-groups, chunks of at least 512 keys) was
  // 1-18 % slower.
  const long long units = (long long)B * Hkv;
  if (units == 0 || Nk == 0) return 1;
  long long want = (512 + units - 1) / units;
  const long long cap = (Nk + 1023) / 1024;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  return (int)want;
}

// Paged caches pass block_table != NULL with page_size / max_pages / num_pages
// and Nk = max_pages * page_size; contiguous caches pass NULL and zeros.
// The decode workspace: the caller's buffer, or (use_scratch) the library's
// own scratch of the current device, for callers that cannot allocate.
enum class Workspace { kCaller, kScratch };

int run_decode(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
               void* o, float* lse, int B, int H, int Hkv, int Nk, int d, float scale,
               int window, int num_splits, void* workspace, size_t workspace_bytes,
               const int* block_table, int page_size, int max_pages, int num_pages,
               void* stream, Workspace ws_kind = Workspace::kCaller) {
  if (B < 0 || H < 1 || Hkv < 1 || Nk < 0) return MIATTN_EINVAL;
  if (H % Hkv != 0) return MIATTN_EINVAL;
  if (window < 0 || !valid_scale(scale)) return MIATTN_EINVAL;
  const int S = resolve_splits(B, Hkv, Nk, num_splits);
  if (S < 0) return S;
  if (d != 64 && d != 128) return MIATTN_EUNSUPPORTED;
  const long long hb = (H / Hkv + 31) / 32;  // blocks of 32 query heads per K/V head
  if ((long long)B * Hkv * hb * S > (long long)INT_MAX || (long long)B * H > (long long)INT_MAX)
    return MIATTN_EUNSUPPORTED;
  // Per-sequence lengths: partial rows are indexed by (share + sequence) <
  // B (S + 1), and the plan counts the batch's key tiles in int.
  if (kv_lens != nullptr && ((long long)B * (S + 1) > (long long)INT_MAX ||
                             (long long)B * ((Nk + 127) / 128) > (long long)INT_MAX / 2))
    return MIATTN_EUNSUPPORTED;
  if (B == 0) return MIATTN_OK;
  if (q == nullptr || o == nullptr) return MIATTN_EINVAL;
  const bool paged = block_table != nullptr;
  if (!paged && Nk > 0 && (k_cache == nullptr || v_cache == nullptr)) return MIATTN_EINVAL;
  if (paged && num_pages > 0 && (k_cache == nullptr || v_cache == nullptr)) return MIATTN_EINVAL;
  const size_t need = miattn::decode_workspace_bytes(B, H, d, S);
  if (ws_kind == Workspace::kScratch) {
    if (need > miattn::kDecodeScratchBytes) return MIATTN_ESCRATCH;
  } else if (workspace == nullptr || workspace_bytes < need) {
    return MIATTN_EWORKSPACE;
  }
  int st = device_status();
  if (st != MIATTN_OK) return st;
  if (ws_kind == Workspace::kScratch) {
    // The scratch copy is the current device's, so the work must run there.
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
      (void)hipGetLastError();
      return MIATTN_ENODEVICE;
    }
    if (stream != nullptr) {
      hipDevice_t sdev = -1;
      if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) {
        (void)hipGetLastError();
        return MIATTN_EINVAL;
      }
      if (sdev != dev) return MIATTN_EINVAL;
    }
    if (miattn::decode_scratch(dev, &workspace) != hipSuccess) {
      (void)hipGetLastError();
      return MIATTN_ELAUNCH;
    }
  }
  DecodeArgs a{q,      k_cache, v_cache, o,         lse,     B,          H,
               Hkv,    Nk,      d,       scale,     window,  S,          workspace,
               kv_lens, block_table, page_size, max_pages, num_pages};
  return launch_status(miattn::launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int Hkv, int Nq, int Nk, int d, float scale, int causal, int window, void* stream) {
  return run_fwd(false, q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, nullptr,
                 stream);
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                 int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
                 void* stream) {
  return run_fwd(true, q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, nullptr,
                 stream);
}

int attn_fwd_fp8(const void* q8, const void* k8, const void* v, void* o, float* lse, int B,
                 int H, int Hkv, int Nq, int Nk, int d, float scale, float q_descale,
                 float k_descale, int causal, int window, void* stream) {
  if (!valid_scale(q_descale) || !valid_scale(k_descale)) return MIATTN_EINVAL;
  const float eff = scale * q_descale * k_descale;
  if (!valid_scale(scale)) return MIATTN_EINVAL;
  if (!valid_scale(eff)) return MIATTN_EUNSUPPORTED;  // the product leaves fp32's range
  int bm = 0, bn = 0;
  if (d == 64 || d == 128) miattn::fwd_bf16_tile_shape(d, &bm, &bn);
  else bm = 1;
  int st = check_fwd(q8, k8, v, o, B, H, Hkv, Nq, Nk, d, eff, causal, window, bm);
  if (st != MIATTN_OK) return st;
  if (B == 0 || Nq == 0) return MIATTN_OK;
  if ((st = device_status()) != MIATTN_OK) return st;
  FwdArgs a{q8, k8, v, o, lse, B, H, Hkv, Nq, Nk, d, eff, causal, window, nullptr,
            nullptr, nullptr, 0, 1};
  return launch_status(miattn::launch_fwd_bf16(a, static_cast<hipStream_t>(stream)));
}

int attn_fwd_tile_counts(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                         int window, int* counts, void* stream) {
  if (counts == nullptr && (long long)B * H * Nq > 0) return MIATTN_EINVAL;
  return run_fwd(false, q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, counts,
                 stream);
}

int attn_fwd_tile_shape(int d, int is_f32, int* block_m, int* block_n) {
  if (block_m == nullptr || block_n == nullptr) return MIATTN_EINVAL;
  if (d != 64 && d != 128) return MIATTN_EUNSUPPORTED;
  if (is_f32) miattn::fwd_f32_tile_shape(d, block_m, block_n);
  else miattn::fwd_bf16_tile_shape(d, block_m, block_n);
  return MIATTN_OK;
}

int attn_decode_num_splits(int B, int Hkv, int Nk, int num_splits) {
  return resolve_splits(B, Hkv, Nk, num_splits);
}

size_t attn_decode_workspace_bytes(int B, int H, int Hkv, int Nk, int d, int num_splits) {
  const int S = resolve_splits(B, Hkv, Nk, num_splits);
  if (S < 0 || B < 0 || H < 1 || d < 1) return 0;
  return miattn::decode_workspace_bytes(B, H, d, S);
}

int attn_decode_splitk(const void* q, const void* k_cache, const void* v_cache, void* o,
                       float* lse, int B, int H, int Hkv, int Nk, int d, float scale, int window,
                       int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return run_decode(q, k_cache, v_cache, nullptr, o, lse, B, H, Hkv, Nk, d, scale, window,
                    num_splits, workspace, workspace_bytes, nullptr, 0, 0, 0, stream);
}

static_assert(miattn::kDecodeScratchBytes == MIATTN_DECODE_SCRATCH_BYTES,
              "the header states the scratch size the library is built with");

int attn_decode_splitk_noalloc(const void* q, const void* k_cache, const void* v_cache,
                               void* o, float* lse, int B, int H, int Hkv, int Nk, int d,
                               float scale, int window, int num_splits, void* stream) {
  return run_decode(q, k_cache, v_cache, nullptr, o, lse, B, H, Hkv, Nk, d, scale, window,
                    num_splits, nullptr, 0, nullptr, 0, 0, 0, stream, Workspace::kScratch);
}

int attn_decode_splitk_varlen(const void* q, const void* k_cache, const void* v_cache,
                              const int* kv_lens, void* o, float* lse, int B, int H, int Hkv,
                              int Nk, int d, float scale, int window, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && kv_lens == nullptr) return MIATTN_EINVAL;
  return run_decode(q, k_cache, v_cache, kv_lens, o, lse, B, H, Hkv, Nk, d, scale, window,
                    num_splits, workspace, workspace_bytes, nullptr, 0, 0, 0, stream);
}

int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int* block_table, const int* kv_lens, void* o, float* lse, int B,
                      int H, int Hkv, int d, int page_size, int num_pages, int max_pages,
                      float scale, int window, int num_splits, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0)
    return MIATTN_EINVAL;
  if (num_pages < 0 || max_pages < 0) return MIATTN_EINVAL;
  const long long nk = (long long)max_pages * page_size;
  if (nk > (long long)INT_MAX) return MIATTN_EUNSUPPORTED;
  if (B > 0 && (kv_lens == nullptr || block_table == nullptr)) return MIATTN_EINVAL;
  return run_decode(q, k_pages, v_pages, kv_lens, o, lse, B, H, Hkv, (int)nk, d, scale, window,
                    num_splits, workspace, workspace_bytes, block_table, page_size, max_pages,
                    num_pages, stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs, int H,
                    int Hkv, int total_q, int total_k, int max_seqlen_q, int d, float scale,
                    int causal, int window, void* stream) {
  return run_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, H, Hkv, total_q,
                        total_k, max_seqlen_q, d, scale, causal, window, nullptr, stream);
}

int attn_fwd_varlen_tile_counts(const void* q, const void* k, const void* v, void* o,
                                float* lse, const int* cu_seqlens_q, const int* cu_seqlens_k,
                                int num_seqs, int H, int Hkv, int total_q, int total_k,
                                int max_seqlen_q, int d, float scale, int causal, int window,
                                int* counts, void* stream) {
  if (counts == nullptr && (long long)num_seqs * H * max_seqlen_q > 0) return MIATTN_EINVAL;
  return run_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, H, Hkv, total_q,
                        total_k, max_seqlen_q, d, scale, causal, window, counts, stream);
}

size_t attn_bwd_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d) {
  if (B < 0 || H < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || d < 1 || H % Hkv != 0) return 0;
  return miattn::bwd_workspace_bytes(B, H, Hkv, Nq, Nk, d);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq,
             int Nk, int d, float scale, int causal, int window, void* workspace,
             size_t workspace_bytes, void* stream) {
  int bm = 0, bn = 0;
  if (d == 64 || d == 128) miattn::fwd_bf16_tile_shape(d, &bm, &bn);
  else bm = 1;
  int st = check_fwd(q, k, v, o, B, H, Hkv, Nq, Nk, d, scale, causal, window, bm);
  if (st != MIATTN_OK) return st;
  const long long nq_elems = (long long)B * H * Nq;
  const long long nk_elems = (long long)B * Hkv * Nk;
  if (nq_elems > 0 && (dout == nullptr || lse == nullptr || dq == nullptr)) return MIATTN_EINVAL;
  if (nk_elems > 0 && (dk == nullptr || dv == nullptr)) return MIATTN_EINVAL;
  if (nk_elems > 0 && (k == nullptr || v == nullptr)) return MIATTN_EINVAL;
  if (nk_elems > 0 && nq_elems > 0 && q == nullptr) return MIATTN_EINVAL;
  // the dK / dV kernel's 1-D grid: one work-group per (batch, head, 128 keys)
  if ((long long)B * H * ((Nk + 127LL) / 128) > (long long)INT_MAX) return MIATTN_EUNSUPPORTED;
  if ((long long)B * Hkv * Nk * d / 8 / 256 > (long long)INT_MAX) return MIATTN_EUNSUPPORTED;
  // the dK / dV kernel streams the Q and dO rows of a head through 32-bit
  // buffer offsets
  if ((long long)Nq * d * 2 > 0xFFFFFFFFLL) return MIATTN_EUNSUPPORTED;
  if (B == 0 || (Nq == 0 && Nk == 0)) return MIATTN_OK;
  const size_t need = miattn::bwd_workspace_bytes(B, H, Hkv, Nq, Nk, d);
  if (workspace == nullptr || workspace_bytes < need) return MIATTN_EWORKSPACE;
  if ((st = device_status()) != MIATTN_OK) return st;
  miattn::BwdArgs a{q,  k, v, o,     dout,   lse,    dq,       dk,  dv, B, H,
                    Hkv, Nq, Nk, d, scale, causal, window, workspace};
  return launch_status(miattn::launch_bwd(a, static_cast<hipStream_t>(stream)));
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs, int H,
                    int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                    int d, float scale, int causal, int window, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || H < 1 || Hkv < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 ||
      max_seqlen_k < 0)
    return MIATTN_EINVAL;
  if (H % Hkv != 0) return MIATTN_EINVAL;
  if (causal != 0 && causal != 1) return MIATTN_EINVAL;
  if (window < 0 || !valid_scale(scale)) return MIATTN_EINVAL;
  if (d != 64 && d != 128) return MIATTN_EUNSUPPORTED;
  if (num_seqs > 0 && (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)) return MIATTN_EINVAL;
  if (total_q > 0 && (q == nullptr || o == nullptr || dout == nullptr || lse == nullptr ||
                      dq == nullptr))
    return MIATTN_EINVAL;
  if (total_k > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return MIATTN_EINVAL;
  const long long nqt = (max_seqlen_q + 127LL) / 128, nkt = (max_seqlen_k + 127LL) / 128;
  if ((long long)num_seqs * H * nqt > (long long)INT_MAX ||
      (long long)num_seqs * H * nkt > (long long)INT_MAX)
    return MIATTN_EUNSUPPORTED;
  if ((long long)total_k * d * 4 > 0xFFFFFFFFLL || (long long)total_q * d * 2 > 0xFFFFFFFFLL ||
      (long long)Hkv * total_k * d / 8 / 256 > (long long)INT_MAX)
    return MIATTN_EUNSUPPORTED;
  if (num_seqs == 0 || (total_q == 0 && total_k == 0)) return MIATTN_OK;
  const size_t need = miattn::bwd_workspace_bytes(1, H, Hkv, total_q, total_k, d);
  if (workspace == nullptr || workspace_bytes < need) return MIATTN_EWORKSPACE;
  int st = device_status();
  if (st != MIATTN_OK) return st;
  miattn::BwdArgs a{q,         k,        v,        o,      dout,   lse,       dq,
                    dk,        dv,       num_seqs, H,      Hkv,    total_q,   total_k,
                    d,         scale,    causal,   window, workspace, cu_seqlens_q,
                    cu_seqlens_k, max_seqlen_q, max_seqlen_k};
  return launch_status(miattn::launch_bwd(a, static_cast<hipStream_t>(stream)));
}

int attn_calib_mfma(int blocks, int iters, float* sink, void* stream) {
  if (blocks < 1 || iters < 1 || sink == nullptr) return MIATTN_EINVAL;
  int st = device_status();
  if (st != MIATTN_OK) return st;
  return launch_status(
      miattn::launch_mfma_ceiling(blocks, iters, sink, static_cast<hipStream_t>(stream)));
}

int attn_calib_read(const void* buf, size_t bytes, unsigned* sink, int blocks, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 || blocks < 1)
    return MIATTN_EINVAL;
  int st = device_status();
  if (st != MIATTN_OK) return st;
  return launch_status(
      miattn::launch_read_ceiling(buf, bytes, sink, blocks, static_cast<hipStream_t>(stream)));
}

const char* attn_strerror(int status) {
  switch (status) {
    case MIATTN_OK: return "success";
    case MIATTN_EINVAL: return "invalid argument";
    case MIATTN_EUNSUPPORTED: return "unsupported configuration";
    case MIATTN_ELAUNCH: return "kernel launch failed";
    case MIATTN_EWORKSPACE: return "workspace missing or too small";
    case MIATTN_ENODEVICE: return "no HIP device available";
    case MIATTN_ESCRATCH:
      return "the call needs more than the library's decode scratch "
             "(MIATTN_DECODE_SCRATCH_BYTES); pass a workspace to attn_decode_splitk instead";
    default: return "unknown status";
  }
}

}  // extern "C"
