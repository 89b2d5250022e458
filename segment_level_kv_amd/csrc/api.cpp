// Host side of the libsx C ABI: argument validation, host planners (RoPE
// table, token classes, realign jobs), workspace sizing and kernel dispatch.
// Nothing here allocates device memory or synchronises a stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <vector>

#include "sx.h"
#include "sx_internal.hpp"

namespace sx {

static thread_local char g_err[512] = "";

sx_status set_error(sx_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sx_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SX_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return SX_OK;
}

sx_status allow_lds(const void* kernel, size_t bytes, const char* what) {
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return set_error(SX_EDEVICE, "%s: LDS request of %zu bytes: %s", what, bytes, hipGetErrorString(e));
  return SX_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace sx

using namespace sx;

namespace {

constexpr int kMaxReq = 8192;

#define SX_REQUIRE(cond, code, ...)                  \
  do {                                               \
    if (!(cond)) return set_error(code, __VA_ARGS__); \
  } while (0)

sx_status check_dims(const sx_dims* d, const char* fn) {
  SX_REQUIRE(d, SX_EINVAL, "%s: dims is NULL", fn);
  SX_REQUIRE(d->dtype == SX_F32 || d->dtype == SX_BF16, SX_EUNSUPPORTED, "%s: dtype %d not supported",
             fn, d->dtype);
  SX_REQUIRE(d->page_size == 16, SX_EUNSUPPORTED, "%s: page_size must be 16 (got %d)", fn, d->page_size);
  SX_REQUIRE(d->n_kv_heads > 0 && d->n_q_heads > 0 && d->n_q_heads % d->n_kv_heads == 0, SX_EINVAL,
             "%s: n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", fn, d->n_q_heads,
             d->n_kv_heads);
  SX_REQUIRE(d->n_q_heads / d->n_kv_heads <= 8, SX_EUNSUPPORTED, "%s: more than 8 query heads per kv head", fn);
  SX_REQUIRE(d->hidden > 0, SX_EINVAL, "%s: hidden must be positive", fn);
  if (d->dtype == SX_BF16) {
    SX_REQUIRE(d->head_dim == 128, SX_EUNSUPPORTED, "%s: bf16 path needs head_dim 128 (got %d)", fn,
               d->head_dim);
    SX_REQUIRE(d->hidden % 64 == 0, SX_EUNSUPPORTED, "%s: bf16 path needs hidden %% 64 == 0", fn);
  } else {
    SX_REQUIRE(d->head_dim == 64 || d->head_dim == 128, SX_EUNSUPPORTED,
               "%s: fp32 path needs head_dim 64 or 128 (got %d)", fn, d->head_dim);
    SX_REQUIRE(d->hidden <= 8192, SX_EUNSUPPORTED, "%s: fp32 path needs hidden <= 8192", fn);
  }
  return SX_OK;
}

sx_status check_layout(const sx_layout* L, const char* fn) {
  SX_REQUIRE(L, SX_EINVAL, "%s: layout is NULL", fn);
  SX_REQUIRE(L->n_req >= 1 && L->n_req <= kMaxReq, SX_EINVAL, "%s: n_req must be in [1, %d]", fn, kMaxReq);
  SX_REQUIRE(L->n_tok >= 0, SX_EINVAL, "%s: n_tok must be >= 0", fn);
  SX_REQUIRE(L->max_pages >= 0, SX_EINVAL, "%s: max_pages must be >= 0", fn);
  SX_REQUIRE(L->n_tok == 0 || L->max_pages > 0, SX_EINVAL,
             "%s: max_pages is 0 but the batch has %d tokens", fn, L->n_tok);
  SX_REQUIRE(L->seq_start && L->block_table, SX_EINVAL, "%s: seq_start/block_table is NULL", fn);
  SX_REQUIRE(L->rope_tab && L->rope_len > 0, SX_EINVAL, "%s: rope_tab missing", fn);
  return SX_OK;
}

sx_status check_pages(const sx_pages* p, const char* fn, const char* which) {
  SX_REQUIRE(p, SX_EINVAL, "%s: %s pages is NULL", fn, which);
  SX_REQUIRE(p->k && p->v, SX_EINVAL, "%s: %s pages has a NULL pool", fn, which);
  SX_REQUIRE(p->n_pages >= 0, SX_EINVAL, "%s: %s n_pages < 0", fn, which);
  return SX_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

#define SX_TRY(expr)                     \
  do {                                   \
    const sx_status st_ = (expr);        \
    if (st_ != SX_OK) return st_;        \
  } while (0)

}  // namespace

extern "C" {

const char* sx_last_error(void) { return g_err; }

sx_status sx_rope_table(double theta, int32_t head_dim, int32_t n_pos, float* tab_h) {
  SX_REQUIRE(tab_h, SX_EINVAL, "sx_rope_table: tab_h is NULL");
  SX_REQUIRE(theta > 0 && std::isfinite(theta), SX_EINVAL, "sx_rope_table: theta must be > 0");
  SX_REQUIRE(head_dim > 0 && head_dim % 2 == 0, SX_EINVAL, "sx_rope_table: head_dim must be even and > 0");
  SX_REQUIRE(n_pos > 0, SX_EINVAL, "sx_rope_table: n_pos must be > 0");
  const int half = head_dim / 2;
  std::vector<double> om(half);
  for (int e = 0; e < half; ++e) om[e] = std::pow(theta, -2.0 * e / head_dim);
  for (int64_t m = 0; m < n_pos; ++m)
    for (int e = 0; e < half; ++e) {
      const double a = (double)m * om[e];
      tab_h[(m * half + e) * 2 + 0] = (float)std::cos(a);
      tab_h[(m * half + e) * 2 + 1] = (float)std::sin(a);
    }
  return SX_OK;
}

sx_status sx_plan_layout(int32_t n_req, const int32_t* piece_start_h, const int32_t* piece_reuse_h,
                         const int32_t* piece_len_h, const int32_t* ratio_num_h,
                         const int32_t* ratio_den_h, int32_t fallback_tokens,
                         int32_t overflow_tokens, int32_t n_tok_cap, int32_t* seq_start_h,
                         uint8_t* tok_class_h, int32_t* sq_rows_h, int32_t* sq_start_h,
                         int32_t* n_cand_h, int32_t* k_h) {
  SX_REQUIRE(n_req >= 1, SX_EINVAL, "sx_plan_layout: n_req must be >= 1");
  SX_REQUIRE(piece_start_h && piece_reuse_h && piece_len_h && ratio_num_h && ratio_den_h &&
                 seq_start_h && tok_class_h && sq_rows_h && sq_start_h && n_cand_h && k_h,
             SX_EINVAL, "sx_plan_layout: NULL argument");
  SX_REQUIRE(fallback_tokens >= 0, SX_EINVAL, "sx_plan_layout: fallback_tokens < 0");
  SX_REQUIRE(overflow_tokens >= 0, SX_EINVAL, "sx_plan_layout: overflow_tokens < 0");
  SX_REQUIRE(piece_start_h[0] == 0, SX_EINVAL, "sx_plan_layout: piece_start_h[0] must be 0");
  // validate everything before writing any output
  int64_t total = 0;
  for (int r = 0; r < n_req; ++r) {
    SX_REQUIRE(piece_start_h[r + 1] >= piece_start_h[r], SX_EINVAL,
               "sx_plan_layout: piece_start_h not ascending at request %d", r);
    SX_REQUIRE(ratio_den_h[r] > 0 && ratio_num_h[r] >= 0 && ratio_num_h[r] <= ratio_den_h[r],
               SX_EINVAL, "sx_plan_layout: ratio of request %d not a fraction in [0,1]", r);
    for (int p = piece_start_h[r]; p < piece_start_h[r + 1]; ++p) {
      SX_REQUIRE(piece_len_h[p] >= 0, SX_EINVAL, "sx_plan_layout: negative length of piece %d", p);
      total += piece_len_h[p];
    }
  }
  SX_REQUIRE(total <= n_tok_cap, SX_EINVAL, "sx_plan_layout: %lld tokens exceed n_tok_cap %d",
             (long long)total, n_tok_cap);
  int tok = 0, nsq = 0;
  seq_start_h[0] = 0;
  sq_start_h[0] = 0;
  for (int r = 0; r < n_req; ++r) {
    const int t0 = tok;
    int last_reuse_len = -1;   // length of the last non-empty piece if it is reused
    int prev_kind = -1;        // previous non-empty piece: -1 none, 0 new, 1 reused
    int prev_len = 0;
    for (int p = piece_start_h[r]; p < piece_start_h[r + 1]; ++p) {
      const int L = piece_len_h[p];
      if (L == 0) continue;
      const int kind = piece_reuse_h[p] ? 1 : 0;
      const uint8_t cls = kind ? 0 : 1;
      for (int j = 0; j < L; ++j) tok_class_h[tok + j] = cls;
      // Overflow (§3.3): one block of each reused neighbour of a new run
      // joins the Sparse-Q set -- the block ending at a new run's start and
      // the block starting right after it.
      if (overflow_tokens > 0 && prev_kind >= 0 && prev_kind != kind) {
        if (kind == 0) {   // reused piece, then this new one
          const int m = prev_len < overflow_tokens ? prev_len : overflow_tokens;
          for (int j = tok - m; j < tok; ++j) tok_class_h[j] = 1;
        } else {           // new run, then this reused piece
          const int m = L < overflow_tokens ? L : overflow_tokens;
          for (int j = tok; j < tok + m; ++j) tok_class_h[j] = 1;
        }
      }
      tok += L;
      prev_kind = kind;
      prev_len = L;
      last_reuse_len = kind ? L : -1;
    }
    if (last_reuse_len > 0) {   // tail fallback: last tokens of the final reused piece probe
      const int m = last_reuse_len < fallback_tokens ? last_reuse_len : fallback_tokens;
      for (int j = tok - m; j < tok; ++j) tok_class_h[j] = 1;
    }
    int n_cand = 0;
    for (int j = t0; j < tok; ++j) {
      if (tok_class_h[j] == 1) sq_rows_h[nsq++] = j;
      else ++n_cand;
    }
    seq_start_h[r + 1] = tok;
    sq_start_h[r + 1] = nsq;
    n_cand_h[r] = n_cand;
    k_h[r] = (int32_t)(((int64_t)ratio_num_h[r] * n_cand) / ratio_den_h[r]);
  }
  return SX_OK;
}

int32_t sx_realign_jobs_bound(const sx_segment* segs_h, int32_t n_segs, int32_t page_size) {
  if (!segs_h || n_segs <= 0 || page_size <= 0) return 0;
  int64_t n = 0;
  for (int s = 0; s < n_segs; ++s)
    // pieces <= 1 + page crossings on the source side + crossings on the
    // destination side; each side crosses at most (len + ps - 2) / ps times.
    if (segs_h[s].len > 0) n += 1 + 2 * (((int64_t)segs_h[s].len + page_size - 2) / page_size);
  return n > INT32_MAX ? INT32_MAX : (int32_t)n;
}

sx_status sx_plan_realign(const sx_segment* segs_h, int32_t n_segs, const int32_t* src_page_ids_h,
                          int32_t n_src_ids, const int32_t* block_table_h, int32_t n_req,
                          int32_t max_pages, int32_t page_size, const int32_t* pos_offset_h,
                          sx_realign_job* jobs_h, int32_t max_jobs, int32_t* n_jobs_h) {
  SX_REQUIRE(n_jobs_h, SX_EINVAL, "sx_plan_realign: n_jobs_h is NULL");
  *n_jobs_h = 0;
  SX_REQUIRE(n_segs >= 0, SX_EINVAL, "sx_plan_realign: n_segs < 0");
  if (n_segs == 0) return SX_OK;
  SX_REQUIRE(segs_h && src_page_ids_h && block_table_h && jobs_h, SX_EINVAL,
             "sx_plan_realign: NULL argument");
  SX_REQUIRE(page_size == 16, SX_EUNSUPPORTED, "sx_plan_realign: page_size must be 16");
  int n = 0;
  for (int s = 0; s < n_segs; ++s) {
    const sx_segment& sg = segs_h[s];
    SX_REQUIRE(sg.req >= 0 && sg.req < n_req, SX_EINVAL, "sx_plan_realign: segment %d: bad request", s);
    SX_REQUIRE(sg.len >= 0 && sg.dst_start >= 0 && sg.src_slot0 >= 0 && sg.src_slot0 < page_size &&
                   sg.src_pages_off >= 0,
               SX_EINVAL, "sx_plan_realign: segment %d: negative or out-of-page field", s);
    const int64_t src_pages_needed = ((int64_t)sg.src_slot0 + sg.len + page_size - 1) / page_size;
    SX_REQUIRE(sg.len == 0 || sg.src_pages_off + src_pages_needed <= n_src_ids, SX_EINVAL,
               "sx_plan_realign: segment %d runs past the source page ids", s);
    SX_REQUIRE(sg.len == 0 || ((int64_t)sg.dst_start + sg.len + page_size - 1) / page_size <= max_pages,
               SX_EINVAL, "sx_plan_realign: segment %d runs past its block table row", s);
    const int delta = sg.dst_start + (pos_offset_h ? pos_offset_h[sg.req] : 0) - sg.p_src;
    int j = 0;
    while (j < sg.len) {
      const int ss = sg.src_slot0 + j, ds = sg.dst_start + j;
      const int src_room = page_size - ss % page_size, dst_room = page_size - ds % page_size;
      int cnt = sg.len - j;
      if (cnt > src_room) cnt = src_room;
      if (cnt > dst_room) cnt = dst_room;
      SX_REQUIRE(n < max_jobs, SX_EINVAL, "sx_plan_realign: more than max_jobs (%d) jobs", max_jobs);
      sx_realign_job& jb = jobs_h[n++];
      jb.src_page = src_page_ids_h[sg.src_pages_off + ss / page_size];
      jb.dst_page = block_table_h[(size_t)sg.req * max_pages + ds / page_size];
      jb.src_slot = ss % page_size;
      jb.dst_slot = ds % page_size;
      jb.n_tok = cnt;
      jb.delta = delta;
      j += cnt;
    }
  }
  *n_jobs_h = n;
  return SX_OK;
}

size_t sx_workspace_bytes(int32_t op, const sx_dims* dims, int32_t n_tok, int32_t n_rows, int32_t n_req) {
  if (!dims || n_tok < 0 || n_rows < 0 || n_req < 0) return 0;
  switch (op) {
    case SX_OP_SELECT: return select_ws_bytes(*dims, n_tok, n_rows, n_req);
    case SX_OP_TOPK: return topk_ws_bytes(n_tok, n_req);
    case SX_OP_SPARSE_ATTN: return attn_ws_bytes(*dims, n_rows, n_req, true);
    case SX_OP_FULL_ATTN: return attn_ws_bytes(*dims, n_tok, n_req, true);
    case SX_OP_DECODE: return decode_ws_bytes(*dims, n_tok, n_req);
    default: return 0;
  }
}

sx_status sx_rope_realign(const sx_dims* dims, const sx_layout* lay, const sx_pages* src,
                          const sx_pages* dst, const sx_realign_job* jobs, int32_t n_jobs,
                          void* stream) {
  const char* fn = "sx_rope_realign";
  SX_TRY(check_dims(dims, fn));
  SX_REQUIRE(lay && lay->rope_tab && lay->rope_len > 0, SX_EINVAL, "%s: layout/rope_tab missing", fn);
  SX_TRY(check_pages(src, fn, "src"));
  SX_TRY(check_pages(dst, fn, "dst"));
  SX_REQUIRE(n_jobs >= 0, SX_EINVAL, "%s: n_jobs < 0", fn);
  SX_REQUIRE(n_jobs == 0 || jobs, SX_EINVAL, "%s: jobs is NULL", fn);
  if (debug_enabled() && n_jobs > 0) {
    DebugCheck dc(as_stream(stream), fn);
    dc.jobs(jobs, n_jobs, src->n_pages, dst->n_pages, lay->rope_len);
    SX_TRY(dc.finish());
  }
  return launch_realign(*dims, *lay, *src, *dst, jobs, n_jobs, as_stream(stream));
}

sx_status sx_recompute_kv(const sx_dims* dims, const sx_layout* lay, const void* x,
                          const int32_t* rows, int32_t n_rows, const void* w_qkv,
                          const sx_pages* kv, void* q_out, void* stream) {
  const char* fn = "sx_recompute_kv";
  SX_TRY(check_dims(dims, fn));
  SX_TRY(check_layout(lay, fn));
  SX_TRY(check_pages(kv, fn, "kv"));
  SX_REQUIRE(n_rows >= 0, SX_EINVAL, "%s: n_rows < 0", fn);
  SX_REQUIRE(n_rows == 0 || (x && rows && w_qkv), SX_EINVAL, "%s: x/rows/w_qkv is NULL", fn);
  if (debug_enabled() && n_rows > 0) {
    DebugCheck dc(as_stream(stream), fn);
    dc.layout(*lay, kv->n_pages, true);
    dc.rows(rows, nullptr, n_rows, *lay);
    SX_TRY(dc.finish());
  }
  return launch_recompute(*dims, *lay, x, rows, n_rows, w_qkv, *kv, q_out, as_stream(stream));
}

sx_status sx_sparse_attn(const sx_dims* dims, const sx_layout* lay, const void* q,
                         const int32_t* rows, const int32_t* row_start, int32_t n_rows,
                         const sx_pages* kv, void* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  const char* fn = "sx_sparse_attn";
  SX_TRY(check_dims(dims, fn));
  SX_TRY(check_layout(lay, fn));
  SX_TRY(check_pages(kv, fn, "kv"));
  SX_REQUIRE(n_rows >= 0, SX_EINVAL, "%s: n_rows < 0", fn);
  if (n_rows == 0) return SX_OK;
  SX_REQUIRE(q && rows && row_start && o, SX_EINVAL, "%s: q/rows/row_start/o is NULL", fn);
  const size_t need = sx_workspace_bytes(SX_OP_SPARSE_ATTN, dims, lay->n_tok, n_rows, lay->n_req);
  SX_REQUIRE(need == 0 || (ws && ws_bytes >= need), SX_EWORKSPACE,
             "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : (size_t)0);
  if (debug_enabled()) {
    DebugCheck dc(as_stream(stream), fn);
    dc.layout(*lay, kv->n_pages, false);
    dc.rows(rows, row_start, n_rows, *lay);
    SX_TRY(dc.finish());
  }
  return launch_attention(*dims, *lay, q, nullptr, rows, row_start, n_rows, *kv, o, lse, ws,
                          as_stream(stream));
}

sx_status sx_sparse_attn_plan(const sx_dims* dims, const sx_layout* lay, const int32_t* rows,
                              const int32_t* row_start, int32_t n_rows, void* ws, size_t ws_bytes,
                              void* stream) {
  const char* fn = "sx_sparse_attn_plan";
  SX_TRY(check_dims(dims, fn));
  SX_TRY(check_layout(lay, fn));
  SX_REQUIRE(n_rows >= 0, SX_EINVAL, "%s: n_rows < 0", fn);
  if (n_rows == 0) return SX_OK;
  SX_REQUIRE(rows && row_start, SX_EINVAL, "%s: rows/row_start is NULL", fn);
  const size_t need = sx_workspace_bytes(SX_OP_SPARSE_ATTN, dims, lay->n_tok, n_rows, lay->n_req);
  SX_REQUIRE(need == 0 || (ws && ws_bytes >= need), SX_EWORKSPACE,
             "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : (size_t)0);
  if (debug_enabled()) {
    DebugCheck dc(as_stream(stream), fn);
    dc.layout(*lay, 1 << 30, false);   // the plan reads offsets and rows, not pages
    dc.rows(rows, row_start, n_rows, *lay);
    SX_TRY(dc.finish());
  }
  return launch_attention_plan(*dims, *lay, rows, row_start, n_rows, ws, as_stream(stream));
}

sx_status sx_sparse_attn_run(const sx_dims* dims, const sx_layout* lay, const void* q,
                             const int32_t* rows, int32_t n_rows, const sx_pages* kv, void* o,
                             float* lse, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "sx_sparse_attn_run";
  SX_TRY(check_dims(dims, fn));
  SX_TRY(check_layout(lay, fn));
  SX_TRY(check_pages(kv, fn, "kv"));
  SX_REQUIRE(n_rows >= 0, SX_EINVAL, "%s: n_rows < 0", fn);
  if (n_rows == 0) return SX_OK;
  SX_REQUIRE(q && rows && o, SX_EINVAL, "%s: q/rows/o is NULL", fn);
  const size_t need = sx_workspace_bytes(SX_OP_SPARSE_ATTN, dims, lay->n_tok, n_rows, lay->n_req);
  SX_REQUIRE(need == 0 || (ws && ws_bytes >= need), SX_EWORKSPACE,
             "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : (size_t)0);
  if (debug_enabled()) {
    DebugCheck dc(as_stream(stream), fn);
    dc.layout(*lay, kv->n_pages, false);
    dc.rows(rows, nullptr, n_rows, *lay);
    SX_TRY(dc.finish());
  }
  return launch_attention_run(*dims, *lay, q, nullptr, rows, n_rows, *kv, o, lse, ws, as_stream(stream));
}

sx_status sx_full_attn(const sx_dims* dims, const sx_layout* lay, const void* q, const sx_pages* kv,
                       void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "sx_full_attn";
  SX_TRY(check_dims(dims, fn));
  SX_TRY(check_layout(lay, fn));
  SX_TRY(check_pages(kv, fn, "kv"));
  if (lay->n_tok == 0) return SX_OK;
  SX_REQUIRE(q && o, SX_EINVAL, "%s: q/o is NULL", fn);
  const size_t need = sx_workspace_bytes(SX_OP_FULL_ATTN, dims, lay->n_tok, lay->n_tok, lay->n_req);
  SX_REQUIRE(need == 0 || (ws && ws_bytes >= need), SX_EWORKSPACE,
             "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : (size_t)0);
  if (debug_enabled()) {
    DebugCheck dc(as_stream(stream), fn);
    dc.layout(*lay, kv->n_pages, false);
    SX_TRY(dc.finish());
  }
  return launch_attention(*dims, *lay, q, nullptr, nullptr, lay->seq_start, lay->n_tok, *kv, o, lse,
                          ws, as_stream(stream));
}

sx_status sx_decode_attn(const sx_dims* dims, const sx_layout* lay, const void* q,
                         const sx_pages* kv, void* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  const char* fn = "sx_decode_attn";
  SX_TRY(check_dims(dims, fn));
  SX_REQUIRE(dims->dtype == SX_BF16, SX_EUNSUPPORTED, "%s: only the bf16 path is built", fn);
  SX_TRY(check_layout(lay, fn));
  SX_TRY(check_pages(kv, fn, "kv"));
  SX_REQUIRE(q && o, SX_EINVAL, "%s: q/o is NULL", fn);
  const size_t need = sx_workspace_bytes(SX_OP_DECODE, dims, lay->n_tok, 0, lay->n_req);
  SX_REQUIRE(ws && ws_bytes >= need, SX_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn,
             need, ws ? ws_bytes : (size_t)0);
  if (debug_enabled()) {
    DebugCheck dc(as_stream(stream), fn);
    dc.layout(*lay, kv->n_pages, false);
    SX_TRY(dc.finish());
  }
  return launch_decode(*dims, *lay, q, *kv, o, lse, ws, as_stream(stream));
}

sx_status sx_decode_attn_noalloc(const sx_dims* dims, const sx_layout* lay, const void* q,
                                 const sx_pages* kv, void* o, float* lse, void* stream) {
  const char* fn = "sx_decode_attn_noalloc";
  SX_TRY(check_dims(dims, fn));
  SX_REQUIRE(dims->dtype == SX_BF16, SX_EUNSUPPORTED, "%s: only the bf16 path is built", fn);
  SX_TRY(check_layout(lay, fn));
  SX_TRY(check_pages(kv, fn, "kv"));
  SX_REQUIRE(q && o, SX_EINVAL, "%s: q/o is NULL", fn);
  const size_t need = sx_workspace_bytes(SX_OP_DECODE, dims, lay->n_tok, 0, lay->n_req);
  SX_REQUIRE(need <= decode_noalloc_capacity(), SX_EWORKSPACE,
             "%s: this batch needs %zu bytes of scratch, the static scratch holds %zu "
             "(split the batch, or use sx_decode_attn with a workspace)",
             fn, need, decode_noalloc_capacity());
  if (debug_enabled()) {
    DebugCheck dc(as_stream(stream), fn);
    dc.layout(*lay, kv->n_pages, false);
    SX_TRY(dc.finish());
  }
  void* ws = nullptr;
  SX_TRY(decode_scratch(&ws));
  return launch_decode(*dims, *lay, q, *kv, o, lse, ws, as_stream(stream));
}

sx_status sx_mfma_peak_probe(int32_t n_workgroups, int32_t iters, int32_t random_operands, float* out,
                             void* stream) {
  const char* fn = "sx_mfma_peak_probe";
  SX_REQUIRE(n_workgroups >= 1 && n_workgroups <= (1 << 20), SX_EINVAL, "%s: n_workgroups must be in [1, 2^20]", fn);
  SX_REQUIRE(iters >= 1 && iters <= (1 << 20), SX_EINVAL, "%s: iters must be in [1, 2^20]", fn);
  SX_REQUIRE(out, SX_EINVAL, "%s: out is NULL", fn);
  return launch_mfma_peak(n_workgroups, iters, random_operands ? 1 : 0, out, as_stream(stream));
}

sx_status sx_topk(const float* scores, const uint8_t* tok_class, const int32_t* seq_start,
                  int32_t n_req, int32_t n_tok, const int32_t* k_sel, int32_t* sel_rows, void* ws,
                  size_t ws_bytes, void* stream) {
  const char* fn = "sx_topk";
  SX_REQUIRE(n_req >= 1 && n_req <= kMaxReq, SX_EINVAL, "%s: n_req must be in [1, %d]", fn, kMaxReq);
  SX_REQUIRE(n_tok >= 0, SX_EINVAL, "%s: n_tok < 0", fn);
  SX_REQUIRE(scores && tok_class && seq_start && k_sel && sel_rows, SX_EINVAL, "%s: NULL argument", fn);
  const size_t need = topk_ws_bytes(n_tok, n_req);
  SX_REQUIRE(ws && ws_bytes >= need, SX_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn,
             need, ws ? ws_bytes : (size_t)0);
  return launch_topk(scores, 1, tok_class, seq_start, n_req, n_tok, k_sel, nullptr, sel_rows, nullptr,
                     const_cast<float*>(scores), ws, as_stream(stream));
}

sx_status sx_recompute_kv_realign(const sx_dims* dims, const sx_layout* lay, const void* x,
                                  const int32_t* rows, int32_t n_rows, const void* w_qkv,
                                  const sx_pages* kv, void* q_out, const sx_pages* rsrc,
                                  const sx_pages* rdst, const sx_realign_job* jobs, int32_t n_jobs,
                                  void* stream) {
  const char* fn = "sx_recompute_kv_realign";
  SX_TRY(check_dims(dims, fn));
  SX_TRY(check_layout(lay, fn));
  SX_TRY(check_pages(kv, fn, "kv"));
  SX_TRY(check_pages(rsrc, fn, "rsrc"));
  SX_TRY(check_pages(rdst, fn, "rdst"));
  SX_REQUIRE(n_rows >= 0, SX_EINVAL, "%s: n_rows < 0", fn);
  SX_REQUIRE(n_rows == 0 || (x && rows && w_qkv), SX_EINVAL, "%s: x/rows/w_qkv is NULL", fn);
  SX_REQUIRE(n_jobs >= 0, SX_EINVAL, "%s: n_jobs < 0", fn);
  SX_REQUIRE(n_jobs == 0 || jobs, SX_EINVAL, "%s: jobs is NULL", fn);
  SX_REQUIRE(rdst->k != kv->k && rdst->v != kv->v && rdst->k != kv->v && rdst->v != kv->k, SX_EINVAL,
             "%s: the realign destination must be another pool than kv", fn);
  hipStream_t s = as_stream(stream);
  if (debug_enabled() && (n_rows > 0 || n_jobs > 0)) {
    DebugCheck dc(s, fn);
    if (n_rows > 0) {
      dc.layout(*lay, kv->n_pages, true);
      dc.rows(rows, nullptr, n_rows, *lay);
    }
    if (n_jobs > 0) dc.jobs(jobs, n_jobs, rsrc->n_pages, rdst->n_pages, lay->rope_len);
    SX_TRY(dc.finish());
  }
  return launch_recompute_realign(*dims, *lay, x, rows, n_rows, w_qkv, *kv, q_out, *rsrc, *rdst, jobs,
                                  n_jobs, s);
}

sx_status sx_select_topk(const sx_dims* dims, const sx_layout* lay, const void* q,
                         const int32_t* q_index, const int32_t* sq_rows, const int32_t* sq_start,
                         int32_t n_sq, const float* lse, const sx_pages* kv,
                         const uint8_t* tok_class, const int32_t* k_sel, int32_t* sel_rows,
                         int32_t* act_rows, float* scores, void* ws, size_t ws_bytes,
                         void* stream) {
  const char* fn = "sx_select_topk";
  SX_TRY(check_dims(dims, fn));
  SX_TRY(check_layout(lay, fn));
  SX_TRY(check_pages(kv, fn, "kv"));
  SX_REQUIRE(n_sq >= 0, SX_EINVAL, "%s: n_sq < 0", fn);
  SX_REQUIRE(tok_class && k_sel && sel_rows && sq_start, SX_EINVAL,
             "%s: tok_class/k_sel/sel_rows/sq_start is NULL", fn);
  SX_REQUIRE(n_sq == 0 || (q && sq_rows), SX_EINVAL, "%s: q/sq_rows is NULL", fn);
  const size_t need = sx_workspace_bytes(SX_OP_SELECT, dims, lay->n_tok, n_sq, lay->n_req);
  SX_REQUIRE(ws && ws_bytes >= need, SX_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn,
             need, ws ? ws_bytes : (size_t)0);
  hipStream_t s = as_stream(stream);
  if (debug_enabled()) {
    DebugCheck dc(s, fn);
    dc.layout(*lay, kv->n_pages, false);
    dc.rows(sq_rows, sq_start, n_sq, *lay);
    SX_TRY(dc.finish());
  }
  char* p = static_cast<char*>(ws);
  float* partial = reinterpret_cast<float*>(p);
  p += align256((size_t)score_parts(*dims, lay->n_tok, lay->n_req) * lay->n_tok * sizeof(float));
  float* score_buf = reinterpret_cast<float*>(p);
  p += align256((size_t)lay->n_tok * sizeof(float));
  float* lse_buf = reinterpret_cast<float*>(p);
  p += align256((size_t)n_sq * dims->n_q_heads * sizeof(float));
  void* attn_ws = p;
  const float* lse_use = lse;
  const int32_t* lse_index = q_index;
  if (n_sq > 0 && !lse) {
    // probe pass: log-sum-exp of every Sparse-Q row over keys 0..i
    SX_TRY(launch_attention(*dims, *lay, q, q_index, sq_rows, sq_start, n_sq, *kv, nullptr, lse_buf,
                            attn_ws, s));
    lse_use = lse_buf;
    lse_index = nullptr;
  }
  if (lay->n_tok > 0) {
    // with no Sparse-Q rows the score kernels write zeros (no query is read)
    // the gathered Sparse-Q rows reuse the probe's work-list space (the probe is done)
    SX_TRY(launch_scores(*dims, *lay, q, q_index, sq_rows, sq_start, n_sq, lse_use, lse_index, *kv,
                         partial, attn_ws, s));
  }
  // the top-k records reuse the same space (the score pass is done)
  return launch_topk(partial, score_parts(*dims, lay->n_tok, lay->n_req), tok_class, lay->seq_start,
                     lay->n_req, lay->n_tok, k_sel, sq_start, sel_rows, act_rows,
                     scores ? scores : score_buf, attn_ws, s);
}

}  // extern "C"
