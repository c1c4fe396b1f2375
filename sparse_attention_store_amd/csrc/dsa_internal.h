// dsa_internal.h -- host-side launchers implemented by each kernel file of libdsa.
// The C ABI layer (dsa_abi.hip) validates arguments and then calls these.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct RowsView {        // device rows + host-known shape
  const int32_t* req;
  const int32_t* pos;
  int32_t n, group, max_pos;
};
struct PagesView {
  const int32_t* pt;
  int64_t pt_stride;
  int32_t num_reqs;
  int64_t num_pages;
};

hipError_t launch_quant_fp8(const uint16_t* x, int64_t n_blocks, uint8_t* y, float* scale, hipStream_t s);
hipError_t launch_index_k_store(const uint16_t* k, RowsView tok, PagesView pg, uint8_t* cache,
                                double eps, const double* inv_freq32, hipStream_t s);
hipError_t launch_latent_store(const uint16_t* kv, RowsView tok, PagesView pg, uint8_t* cache, hipStream_t s);

// range (nullable): per-row [min, max] order-preserving keys of the visible logits, merged
// with atomicMin / atomicMax (the caller initialises it).  skip_upto: row groups whose rows
// all have pos + 1 <= skip_upto are not scored and their logits are not written (0: none).
hipError_t launch_indexer_logits(const uint8_t* q8, const float* qs, const float* w, RowsView rows,
                                 PagesView pg, const uint8_t* cache, float* logits, int64_t stride,
                                 uint32_t* range, int32_t skip_upto, hipStream_t s);

size_t topk_workspace_bytes(int32_t R, int64_t stride, int32_t k);
hipError_t launch_topk(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx,
                       void* ws, hipStream_t s);
// Pieces of the top-k used by the fused indexer + top-k entry.
hipError_t launch_topk_init(int32_t R, int32_t k, void* ws, hipStream_t s);
uint32_t* topk_range_ptr(void* ws, int32_t R, int32_t k);
hipError_t launch_topk_from_range(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx,
                                  void* ws, hipStream_t s);

size_t mla_workspace_bytes(int32_t R, int32_t k);
hipError_t launch_sparse_mla(const uint16_t* q, RowsView rows, PagesView pg, const uint8_t* cache,
                             const int32_t* idx, int32_t k, float sm_scale, uint16_t* out, float* lse,
                             void* ws, size_t ws_bytes, bool prefill, hipStream_t s);

// Read-and-clear of each translation unit's device error flag (synchronous).
int take_device_errors_store();
int take_device_errors_indexer();
int take_device_errors_topk();
int take_device_errors_mla();

}  // namespace dsa
