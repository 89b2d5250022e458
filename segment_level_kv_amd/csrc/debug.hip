// Device-side index checks run when the environment variable SX_DEBUG is set
// (to anything but "0").  The index data of a call -- request offsets, the
// block table (the paper's §4.5 scheduler output: block table and slot
// mapping), row lists and realign jobs -- lives on the device, so the host
// cannot validate it before launching.  With SX_DEBUG, each entry point first
// runs the checks below on its stream: they read the index data only (every
// read bounded by the sizes the caller gave), OR what they find into a flag
// word, and the host waits for the stream and reads it.  If a flag is set
// the call returns SX_EDEVICE naming the problem and launches nothing else,
// so a bad index is reported instead of being dereferenced.  Debug mode
// synchronises the stream (it cannot be captured into a graph).
#include <cstdlib>
#include <mutex>

#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {
namespace {

enum : int {
  F_SEQ = 1,     // request offsets not ascending, outside [0, n_tok], or not ending at n_tok
  F_PAGE = 2,    // a block-table entry a request uses is outside [0, n_pages), or too few columns
  F_POS = 4,     // a RoPE position outside [0, rope_len)
  F_ROWS = 8,    // a row outside its request / the batch, not ascending, or bad row offsets
  F_JOB = 16,    // a realign job's page, slot or count out of range
  F_DELTA = 32,  // a realign job with |delta| >= rope_len
};

// The flag word of the checks; each GPU holds its own copy, whose address
// comes from hipGetSymbolAddress once per device.
static __device__ __align__(256) int dbg_flags[64];
constexpr int kMaxDevices = 64;
std::mutex g_dbg_mu;
int* g_dbg_ptr[kMaxDevices] = {};

__device__ __forceinline__ void raise_flag(int* f, int bit) { atomicOr(f, bit); }

__global__ void dbg_clear(int* f) {
  if (threadIdx.x == 0) f[0] = 0;
}

// One thread per request: offsets, the block-table columns its tokens use,
// and (positions != 0) the RoPE positions of its tokens.
__global__ void dbg_layout(sx_layout lay, int n_pages, int positions, int* f) {
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < lay.n_req; r += gridDim.x * blockDim.x) {
    const int a = lay.seq_start[r], b = lay.seq_start[r + 1];
    if (r == 0 && a != 0) raise_flag(f, F_SEQ);
    if (r == lay.n_req - 1 && b != lay.n_tok) raise_flag(f, F_SEQ);
    if (a < 0 || b < a || b > lay.n_tok) {
      raise_flag(f, F_SEQ);
      continue;
    }
    const int len = b - a;
    const int np = (len + kPage - 1) / kPage;
    if (np > lay.max_pages) raise_flag(f, F_PAGE);
    const int32_t* bt = lay.block_table + (size_t)r * lay.max_pages;
    for (int p = 0; p < min(np, lay.max_pages); ++p) {
      const int pg = bt[p];
      if (pg < 0 || pg >= n_pages) {
        raise_flag(f, F_PAGE);
        break;
      }
    }
    if (positions && len > 0) {
      const long long off = lay.pos_offset ? lay.pos_offset[r] : 0;
      if (off < 0 || off + len - 1 >= lay.rope_len) raise_flag(f, F_POS);
    }
  }
}

// Row lists.  grouped != 0: rows grouped by request per row_start (n_req + 1
// offsets from 0 to n_rows), ascending and inside the request's tokens.
// grouped == 0: every row is a token of the batch, in any order.
__global__ void dbg_rows(const int32_t* rows, const int32_t* row_start, int n_rows, sx_layout lay,
                         int grouped, int* f) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int stride = gridDim.x * blockDim.x;
  if (!grouped) {
    for (int m = tid; m < n_rows; m += stride)
      if (rows[m] < 0 || rows[m] >= lay.n_tok) raise_flag(f, F_ROWS);
    return;
  }
  if (tid == 0 && (row_start[0] != 0 || row_start[lay.n_req] != n_rows)) raise_flag(f, F_ROWS);
  for (int r = tid; r < lay.n_req; r += stride) {
    const int a = row_start[r], b = row_start[r + 1];
    if (a < 0 || b < a || b > n_rows) {
      raise_flag(f, F_ROWS);
      continue;
    }
    const int t0 = lay.seq_start[r], t1 = lay.seq_start[r + 1];
    for (int m = a; m < b; ++m) {
      const int t = rows[m];
      if (t < t0 || t >= t1 || (m > a && t <= rows[m - 1])) {
        raise_flag(f, F_ROWS);
        break;
      }
    }
  }
}

__global__ void dbg_jobs(const sx_realign_job* jobs, int n_jobs, int n_src, int n_dst, int rope_len,
                         int* f) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_jobs; i += gridDim.x * blockDim.x) {
    const sx_realign_job jb = jobs[i];
    if (jb.src_page < 0 || jb.src_page >= n_src || jb.dst_page < 0 || jb.dst_page >= n_dst ||
        jb.n_tok < 0 || jb.src_slot < 0 || jb.dst_slot < 0 || jb.src_slot + jb.n_tok > kPage ||
        jb.dst_slot + jb.n_tok > kPage)
      raise_flag(f, F_JOB);
    const long long ad = jb.delta < 0 ? -(long long)jb.delta : jb.delta;
    if (ad >= rope_len) raise_flag(f, F_DELTA);
  }
}

int grid_for(int n) { return n <= 0 ? 1 : min((n + 255) / 256, 1024); }

}  // namespace

bool debug_enabled() {
  const char* v = std::getenv("SX_DEBUG");
  return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

DebugCheck::DebugCheck(hipStream_t stream, const char* fn) : stream_(stream), fn_(fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    status_ = set_error(SX_EDEVICE, "%s (SX_DEBUG): no usable device", fn);
    return;
  }
  std::lock_guard<std::mutex> lock(g_dbg_mu);
  if (!g_dbg_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_flags));
    if (e != hipSuccess || !p) {
      status_ = set_error(SX_EDEVICE, "%s (SX_DEBUG): hipGetSymbolAddress: %s", fn, hipGetErrorString(e));
      return;
    }
    g_dbg_ptr[dev] = static_cast<int*>(p);
  }
  flag_ = g_dbg_ptr[dev];
  dbg_clear<<<1, 64, 0, stream_>>>(flag_);
  status_ = check_launch("SX_DEBUG check");
}

void DebugCheck::layout(const sx_layout& lay, int n_pages, bool positions) {
  if (status_ != SX_OK) return;
  dbg_layout<<<grid_for(lay.n_req), 256, 0, stream_>>>(lay, n_pages, positions ? 1 : 0, flag_);
  status_ = check_launch("SX_DEBUG layout check");
}

void DebugCheck::rows(const int32_t* rows, const int32_t* row_start, int n_rows,
                      const sx_layout& lay) {
  if (status_ != SX_OK || n_rows <= 0) return;
  const int grouped = row_start ? 1 : 0;
  dbg_rows<<<grid_for(grouped ? lay.n_req : n_rows), 256, 0, stream_>>>(rows, row_start, n_rows, lay,
                                                                      grouped, flag_);
  status_ = check_launch("SX_DEBUG row check");
}

void DebugCheck::jobs(const sx_realign_job* jobs, int n_jobs, int n_src, int n_dst, int rope_len) {
  if (status_ != SX_OK || n_jobs <= 0) return;
  dbg_jobs<<<grid_for(n_jobs), 256, 0, stream_>>>(jobs, n_jobs, n_src, n_dst, rope_len, flag_);
  status_ = check_launch("SX_DEBUG job check");
}

sx_status DebugCheck::finish() {
  if (status_ != SX_OK) return status_;
  int h = 0;
  hipError_t e = hipMemcpyAsync(&h, flag_, sizeof(int), hipMemcpyDeviceToHost, stream_);
  if (e == hipSuccess) e = hipStreamSynchronize(stream_);
  if (e != hipSuccess) return set_error(SX_EDEVICE, "%s (SX_DEBUG): %s", fn_, hipGetErrorString(e));
  if (h == 0) return SX_OK;
  return set_error(SX_EDEVICE, "%s (SX_DEBUG): bad device index data:%s%s%s%s%s%s", fn_,
                   (h & F_SEQ) ? " request offsets;" : "", (h & F_PAGE) ? " block-table page id;" : "",
                   (h & F_POS) ? " RoPE position beyond the table;" : "",
                   (h & F_ROWS) ? " row list;" : "", (h & F_JOB) ? " realign job page/slot/count;" : "",
                   (h & F_DELTA) ? " realign delta beyond the RoPE table;" : "");
}

}  // namespace sx
