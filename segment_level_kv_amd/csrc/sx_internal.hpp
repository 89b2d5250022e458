// Host-side internal interface between the C ABI (api.cpp) and the kernel
// launchers (*.hip).  Launchers assume validated arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sx.h"

namespace sx {

// Records `msg` as the calling thread's last error and returns `st`.
sx_status set_error(sx_status st, const char* fmt, ...);
// SX_OK, or SX_EDEVICE with the HIP error text if the last launch failed.
sx_status check_launch(const char* what);

// Lets `kernel` use `bytes` of dynamic LDS (gfx950 has 160 KB per CU).
sx_status allow_lds(const void* kernel, size_t bytes, const char* what);

// Workspace carving (all offsets 256-byte aligned).
size_t align256(size_t x);
// Attention workspace (bf16 path): work list and partial results of key
// chunks; 0 for fp32.  with_o false: log-sum-exp only (no partial outputs).
size_t attn_ws_bytes(const sx_dims& d, int n_rows, int n_req, bool with_o);
size_t topk_ws_bytes(int n_tok, int n_req);
size_t select_ws_bytes(const sx_dims& d, int n_tok, int n_sq, int n_req);

sx_status launch_realign(const sx_dims& dims, const sx_layout& lay, const sx_pages& src,
                         const sx_pages& dst, const sx_realign_job* jobs, int n_jobs,
                         hipStream_t stream);

sx_status launch_recompute(const sx_dims& dims, const sx_layout& lay, const void* x,
                           const int32_t* rows, int n_rows, const void* w_qkv,
                           const sx_pages& kv, void* q_out, hipStream_t stream);
// launch_recompute of kv plus launch_realign of rsrc -> rdst (pages the
// projection does not write), in one launch when the projection leaves
// compute units free.
sx_status launch_recompute_realign(const sx_dims& dims, const sx_layout& lay, const void* x,
                                   const int32_t* rows, int n_rows, const void* w_qkv,
                                   const sx_pages& kv, void* q_out, const sx_pages& rsrc,
                                   const sx_pages& rdst, const sx_realign_job* jobs, int n_jobs,
                                   hipStream_t stream);

// Attention over the paged cache for rows grouped by request.
//   rows == NULL: row m is packed token m (full prefill), row_start = seq_start.
//   q_index (may be NULL): query of row m is q[q_index[m]].
//   o == NULL: only the log-sum-exp is produced (probe pass).
sx_status launch_attention(const sx_dims& dims, const sx_layout& lay, const void* q,
                           const int32_t* q_index, const int32_t* rows,
                           const int32_t* row_start, int n_rows, const sx_pages& kv, void* o,
                           float* lse, void* ws, hipStream_t stream);

// The two halves of launch_attention: the work list over the rows (into ws;
// a no-op for fp32) and the attention over a work list already in ws, built
// for the same rows, layout and dims.
sx_status launch_attention_plan(const sx_dims& dims, const sx_layout& lay, const int32_t* rows,
                                const int32_t* row_start, int n_rows, void* ws, hipStream_t stream);
sx_status launch_attention_run(const sx_dims& dims, const sx_layout& lay, const void* q,
                               const int32_t* q_index, const int32_t* rows, int n_rows,
                               const sx_pages& kv, void* o, float* lse, void* ws,
                               hipStream_t stream);

// Decode attention: one query row per request (its last token), bf16 only.
size_t decode_ws_bytes(const sx_dims& d, int n_tok, int n_req);
sx_status launch_decode(const sx_dims& dims, const sx_layout& lay, const void* q, const sx_pages& kv,
                        void* o, float* lse, void* ws, hipStream_t stream);
// The static scratch of sx_decode_attn_noalloc: its size, and the current
// device's address of it (looked up on the first call per device).
size_t decode_noalloc_capacity();
sx_status decode_scratch(void** ptr);

// Partial score rows the score pass writes ([parts][n_tok]): one per kv head,
// or per query head for bf16 prompts too short to fill the chip with kv-head
// workgroups; the top-k adds them in row order.
int score_parts(const sx_dims& d, int n_tok, int n_req);

// Partial attention-mass scores of the Sparse-Q rows, per score_parts row.
// gather_ws: scores_gather_bytes(dims, n_sq) bytes for the bf16 path.
size_t scores_gather_bytes(const sx_dims& d, int n_sq);
sx_status launch_scores(const sx_dims& dims, const sx_layout& lay, const void* q,
                        const int32_t* q_index, const int32_t* sq_rows, const int32_t* sq_start,
                        int n_sq, const float* lse, const int32_t* lse_index,
                        const sx_pages& kv, float* partial, void* gather_ws, hipStream_t stream);

// Top-k on the sum over `n_parts` partial score rows ([n_parts][n_tok]).
sx_status launch_topk(const float* partial, int n_parts, const uint8_t* tok_class,
                      const int32_t* seq_start, int n_req, int n_tok, const int32_t* k_sel,
                      const int32_t* sq_start, int32_t* sel_rows, int32_t* act_rows,
                      float* scores_out, void* ws, hipStream_t stream);

// SX_DEBUG device-side index checks (debug.hip).  debug_enabled(): the
// environment variable SX_DEBUG is set to anything but "0".  A DebugCheck
// clears its flag word on `stream`, each check enqueues a kernel that reads
// the index data and ORs flags in, and finish() waits for the stream and
// returns SX_EDEVICE (with the text in sx_last_error) if a flag is set.
bool debug_enabled();
class DebugCheck {
 public:
  DebugCheck(hipStream_t stream, const char* fn);
  // request offsets and the block-table columns each request's tokens use;
  // positions: also the RoPE positions of every token
  void layout(const sx_layout& lay, int n_pages, bool positions);
  // row_start != NULL: rows grouped by request, ascending inside it;
  // row_start == NULL: every row a token of the batch
  void rows(const int32_t* rows, const int32_t* row_start, int n_rows, const sx_layout& lay);
  void jobs(const sx_realign_job* jobs, int n_jobs, int n_src_pages, int n_dst_pages, int rope_len);
  sx_status finish();

 private:
  hipStream_t stream_;
  const char* fn_;
  int* flag_ = nullptr;
  sx_status status_ = SX_OK;
};

// Back-to-back bf16 MFMAs on every compute unit (measured-peak probe).
sx_status launch_mfma_peak(int n_workgroups, int iters, int random_operands, float* out, hipStream_t stream);

}  // namespace sx
