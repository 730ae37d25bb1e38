// Host-side launchers of the libmiattn kernels. Arguments reaching these
// functions have already been validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace miattn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  int causal, window;
  int* counts;  // optional per-work-group (tiles loaded, tiles masked)
  // Packed documents (null for fixed-length calls): B documents whose query
  // and key rows are [cu_q[b], cu_q[b+1]) and [cu_k[b], cu_k[b+1]) of one
  // packed sequence of Nq query rows and Nk key rows; max_q is at least every
  // document's query count.
  const int* cu_q;
  const int* cu_k;
  int max_q;
  // fp8 e4m3 q and k (the scale already includes both descales); v stays bf16.
  int fp8;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Nk, d;
  float scale;
  int window;
  int splits;
  void* workspace;
  // Per-sequence cache lengths in [0, Nk] (null: every sequence holds Nk keys).
  const int* kv_lens;
  // Paged cache (null: contiguous [B, Hkv, Nk, d] caches): k, v are page
  // pools [num_pages, Hkv, page_size, d], block_table is [B, max_pages], and
  // Nk = max_pages * page_size. page_size is a power of two.
  const int* block_table;
  int page_size, max_pages, num_pages;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  int causal, window;
  void* workspace;
  // Packed documents (null for fixed-length calls): as FwdArgs; max_q / max_k
  // bound every document's query / key count. Nq, Nk are the packed totals.
  const int* cu_q;
  const int* cu_k;
  int max_q, max_k;
};

// Query-tile rows / key-tile columns of the bf16 and fp32 forward kernels.
void fwd_bf16_tile_shape(int d, int* block_m, int* block_n);
void fwd_f32_tile_shape(int d, int* block_m, int* block_n);

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);

// Partials layout inside the workspace: O_s fp32 [B, H, S, d], then lse_s fp32 [B, H, S].
size_t decode_workspace_bytes(int B, int H, int d, int splits);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Size of the library's own decode scratch (the no-allocation decode entry
// point); must equal MIATTN_DECODE_SCRATCH_BYTES in miattn.h.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
// Device address of `device`'s copy of the decode scratch, resolved once per
// device; `device` must be the current device on the first call for it.
hipError_t decode_scratch(int device, void** ptr);

// Backward: workspace = D [B, H, Nq] fp32 (256-byte aligned size), then,
// when H > Hkv, fp32 dK and dV partials [B, H, Nk, d] each.
size_t bwd_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

// Ceiling probes (calib.hip).
hipError_t launch_mfma_ceiling(int blocks, int iters, float* sink, hipStream_t stream);
hipError_t launch_read_ceiling(const void* buf, size_t bytes, unsigned* sink, int blocks,
                               hipStream_t stream);

bool log_enabled();

}  // namespace miattn
