// Causal GQA attention of the active rows over the mixed paged KV cache
// (SparseX paper §3.2: Sparse-Q rows attend to all available keys at their
// true positions; §3.4: full attention before the threshold, Sparse-Q plus
// selected rows after it; §4.5 last paragraph: reused blocks are read through
// the block table, recomputed tokens take the normal attention path).
//
// bf16 path (gfx950)
// ------------------
// Work unit: one kv head g and one query tile of (row, head) pairs: M
// consecutive active rows of one request times the G query heads of g
// (M = 256 / G, so a tile is at most 256 pairs: 8 waves of 32, two waves per
// SIMD).  Tiles are split along the key axis into chunks only when there are
// fewer tiles than compute units; each chunk is one workgroup.  A small
// single-workgroup kernel builds the list of (tile, key chunk) items on the
// device (the active rows are device data) and orders it longest first; a
// merge kernel combines the chunks of split tiles in chunk order, so results
// do not depend on scheduling.
//
// Per 32-key sub-block and wave (32 pairs):
//   S^T[key][pair] = K . Q^T    8 x v_mfma_f32_32x32x16_bf16 (one chain)
//   online softmax over the key axis, which lies inside a lane (16 keys per
//   lane and pair, the other 16 in the partner lane half)
//   O^T[d][pair] += V^T . P^T   8 x v_mfma_f32_32x32x16_bf16
// Q, O, S and P all live in VGPRs (no AGPR copies, no scratch).  Keys are
// permuted inside each 32-key sub-block when K is read from LDS so that the
// S^T accumulators are directly the B operand of the PV product.  A step
// issues PV of sub-block j, QK^T of j+2 and the softmax of j+1, which are
// independent, as one scheduling region.  The running maximum is raised
// only when a block's maximum exceeds it by more than 2^8 (in the exp2
// domain), so O is rarely rescaled; exp2 arguments then stay below 8.
// K/V stream through a 4-stage LDS ring of 64-key stages (global -> LDS
// directly, one barrier per stage); the page ids of a stage are
// wave-uniform and come through the scalar cache.  Workgroup b takes kv head
// b % Hkv: with 8 kv heads each XCD streams one head's K/V through its own
// L2.  Final outputs leave through LDS as whole 256-byte rows.
#include <type_traits>

#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

namespace {

constexpr int KB = 64;                 // keys per block
constexpr int NSTAGE = 4;              // LDS ring depth (copies issued 3 stages ahead)
constexpr int PAIRS = 256;             // (row, head) pairs per workgroup
constexpr int kTargetItems = 256;      // work items aimed for (one per CU); tiles are split only below it
constexpr int kMinChunk = 1024;        // shortest key chunk of a split tile
constexpr int kBuildThreads = 1024;
constexpr int kSortBuckets = 2048;     // item length buckets (64 keys each)
constexpr int kFullKeys = 1024;        // sort keys for full chunks (by chunk index)

struct Stage {
  uint16_t k[KB][128];        // 64 key rows, 16-byte chunks XOR-swizzled by row
  uint16_t v[4][128][16];     // 4 V page-heads [d][slot], halves swizzled by d
};

// One workgroup's work: query rows [row0, row0 + nrows) (indices into the
// row list) of request req, keys [k0, k1).  slot < 0: the tile is not split
// and the workgroup writes the final output; otherwise partial results go to
// partial slot `slot`.
struct AttnItem {
  int32_t req, row0, nrows, k0, k1, slot, pad0, pad1;
};
struct MergeTile {
  int32_t row0, nrows, slot0, n_chunks;
};
struct TileInfo {
  int32_t req, row0, nrows, pmin, pmax, n_chunks, item0, slot0;
};

int rows_per_tile(int G) { return PAIRS / G; }
int items_per_head(int hkv) { return (kTargetItems + hkv - 1) / hkv; }

struct WsLayout {
  size_t counters, tiles, items, merges, part_ml, part_o, total;
  int max_tiles, max_items;
};

WsLayout ws_layout(int n_rows, int n_req, int G, int hkv, bool with_o) {
  WsLayout w;
  const int M = rows_per_tile(G);
  w.max_tiles = (n_rows + M - 1) / M + n_req;
  w.max_items = 2 * w.max_tiles + items_per_head(hkv);
  size_t off = 0;
  w.counters = off; off += align256(4 * sizeof(int32_t));
  w.tiles = off;    off += align256((size_t)w.max_tiles * sizeof(TileInfo));
  w.items = off;    off += align256((size_t)w.max_items * sizeof(AttnItem));
  w.merges = off;   off += align256((size_t)w.max_tiles * sizeof(MergeTile));
  w.part_ml = off;  off += align256((size_t)w.max_items * hkv * PAIRS * 4 * sizeof(float));
  w.part_o = off;
  if (with_o) off += align256((size_t)w.max_items * hkv * PAIRS * 128 * sizeof(uint16_t));
  w.total = off;
  return w;
}

// Block-wide exclusive scan over kBuildThreads threads; *total gets the sum.
__device__ int build_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < kBuildThreads / 64; ++i) {
    const int s = sh[i];
    before += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Builds the (tile, key chunk) work list.  One workgroup.
//   rows == NULL: row m is packed token m.  Positions are row - seq_start[r].
// Counters: [0] items, [1] merge tiles.  Dynamic LDS: (n_req + 1) ints.
__global__ __launch_bounds__(kBuildThreads) void build_work(
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ seq_start, int n_req, int n_rows, int M, int items_target,
    int max_tiles, int max_items, int allow_split, TileInfo* __restrict__ tiles,
    AttnItem* __restrict__ items, MergeTile* __restrict__ merges, int32_t* __restrict__ counters) {
  extern __shared__ int roff[];              // first tile of each request
  __shared__ int sh_scan[kBuildThreads / 64];
  __shared__ int hist[kFullKeys + kSortBuckets];
  __shared__ long long s_work[kBuildThreads / 64];
  const int tid = threadIdx.x;

  // ---- tiles per request -> offsets ---------------------------------------------
  int n_tiles = 0;
  for (int r0 = 0; r0 < n_req; r0 += kBuildThreads) {
    const int r = r0 + tid;
    int c = 0;
    if (r < n_req) {
      const int a = max(row_start[r], 0), b = min(row_start[r + 1], n_rows);
      c = b > a ? (b - a + M - 1) / M : 0;
    }
    int tot;
    const int off = n_tiles + build_scan(c, sh_scan, &tot);
    if (r < n_req) roff[r] = off;
    n_tiles += tot;
  }
  if (tid == 0) roff[n_req] = n_tiles;
  __syncthreads();
  n_tiles = min(n_tiles, max_tiles);

  // ---- one thread per tile --------------------------------------------------------
  long long work = 0;
  for (int t = tid; t < n_tiles; t += kBuildThreads) {
    int lo = 0, hi = n_req - 1;              // request r with roff[r] <= t < roff[r+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (roff[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int a = max(row_start[r], 0), b = min(row_start[r + 1], n_rows);
    const int s0 = seq_start[r];
    const int row0 = a + (t - roff[r]) * M;
    const int nr = min(M, b - row0);
    const int pmin = (rows ? rows[row0] : row0) - s0;
    const int pmax = (rows ? rows[row0 + nr - 1] : row0 + nr - 1) - s0;
    TileInfo ti_;
    ti_.req = r;
    ti_.row0 = row0;
    ti_.nrows = nr;
    ti_.pmin = max(pmin, 0);
    ti_.pmax = max(pmax, ti_.pmin);
    ti_.n_chunks = 1;
    ti_.item0 = 0;
    ti_.slot0 = -1;
    tiles[t] = ti_;
    work += (long long)ti_.pmax + 1;
  }
  // total key work -> chunk length
  {
    long long x = work;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if ((tid & 63) == 0) s_work[tid >> 6] = x;
  }
  __syncthreads();   // tiles[] written by this workgroup are visible after the barrier
  long long total_work = 0;
  for (int i = 0; i < kBuildThreads / 64; ++i) total_work += s_work[i];
  const bool split = allow_split && n_tiles < items_target;
  long long ck = split ? (total_work + items_target - 1) / items_target : 0x3fffffff;
  ck = ((ck + KB - 1) / KB) * KB;
  if (ck < kMinChunk) ck = kMinChunk;
  const int chunk = (int)min(ck, 0x3fffffffLL);

  // ---- chunks per tile, item and slot offsets -------------------------------------
  int item_base = 0, slot_base = 0, merge_base = 0;
  for (int t0 = 0; t0 < n_tiles; t0 += kBuildThreads) {
    const int t = t0 + tid;
    int nc = 0;
    if (t < n_tiles) nc = split ? (tiles[t].pmax + chunk) / chunk : 1;   // ceil((pmax+1)/chunk)
    int tot_i, tot_s, tot_m;
    const int io = item_base + build_scan(nc, sh_scan, &tot_i);
    const int so = slot_base + build_scan(nc > 1 ? nc : 0, sh_scan, &tot_s);
    const int mo = merge_base + build_scan(nc > 1 ? 1 : 0, sh_scan, &tot_m);
    if (t < n_tiles) {
      tiles[t].n_chunks = nc;
      tiles[t].item0 = io;
      tiles[t].slot0 = nc > 1 ? so : -1;
      if (nc > 1) {
        MergeTile mt;
        mt.row0 = tiles[t].row0;
        mt.nrows = tiles[t].nrows;
        mt.slot0 = so;
        mt.n_chunks = nc;
        merges[mo] = mt;
      }
    }
    item_base += tot_i;
    slot_base += tot_s;
    merge_base += tot_m;
  }
  const int n_items = min(item_base, max_items);

  // ---- items, counting-sorted ------------------------------------------------------
  // Chunks of a split tile sit on a grid shared by all tiles: [c*chunk,
  // (c+1)*chunk) up to pmax.  A chunk may lie wholly past some rows of the
  // tile (rows far apart in position); those rows get an empty partial
  // (m = -inf, l = 0) that the merge weighs with 0.  Order: full chunks
  // first, by chunk index (the workgroups running together on an XCD then
  // stream the same keys of one kv head, which its L2 shares), then the
  // other items longest first.
  for (int i = tid; i < kFullKeys + kSortBuckets; i += kBuildThreads) hist[i] = 0;
  __syncthreads();
  auto chunk_range = [&](const TileInfo& T, int c, int& k0, int& k1) {
    k0 = c * chunk;
    k1 = min(k0 + chunk, T.pmax + 1);
  };
  auto sort_key = [&](const TileInfo& T, int c, int k0, int k1) {
    if (T.n_chunks > 1 && k1 - k0 == chunk) return min(c, kFullKeys - 1);
    return kFullKeys + kSortBuckets - 1 - min((k1 - k0 - 1) / KB, kSortBuckets - 1);
  };
  for (int t = tid; t < n_tiles; t += kBuildThreads) {
    const TileInfo T = tiles[t];
    for (int c = 0; c < T.n_chunks; ++c) {
      int k0, k1;
      chunk_range(T, c, k0, k1);
      atomicAdd(&hist[sort_key(T, c, k0, k1)], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the histogram
  {
    constexpr int PER = (kFullKeys + kSortBuckets) / kBuildThreads;
    static_assert(PER * kBuildThreads == kFullKeys + kSortBuckets, "histogram split");
    int loc[PER], s = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      loc[i] = hist[tid * PER + i];
      s += loc[i];
    }
    int tot;
    int pre = build_scan(s, sh_scan, &tot);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      hist[tid * PER + i] = pre;
      pre += loc[i];
    }
  }
  __syncthreads();
  for (int t = tid; t < n_tiles; t += kBuildThreads) {
    const TileInfo T = tiles[t];
    for (int c = 0; c < T.n_chunks; ++c) {
      int k0, k1;
      chunk_range(T, c, k0, k1);
      const int pos = atomicAdd(&hist[sort_key(T, c, k0, k1)], 1);
      if (pos >= max_items) continue;
      AttnItem it;
      it.req = T.req;
      it.row0 = T.row0;
      it.nrows = T.nrows;
      it.k0 = k0;
      it.k1 = k1;
      it.slot = T.n_chunks > 1 ? T.slot0 + c : -1;
      it.pad0 = T.pmin;
      it.pad1 = T.pmax;
      items[pos] = it;
    }
  }
  if (tid == 0) {
    counters[0] = n_items;
    counters[1] = merge_base;
  }
}

// max / sum of a value over the two lane halves (lanes l and l^32), in every
// lane: v_permlane32_swap exchanges the halves without going through LDS.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt with at most VM vector-memory operations of this wave still in
// flight, then the workgroup barrier.  The stage copies (global_load_lds)
// write LDS asynchronously and are tracked only by vmcnt, which the barrier
// itself does not wait for.  LDS reads may still be in flight: the ones a
// wave issues just before the barrier load the next step's operands from
// stages that stay resident, and every read of the slot the copies after
// the barrier overwrite was consumed by an MFMA, hence complete, before the
// wave reached it (waiting for them here as well cost 2% of the loop).
// Written as one asm block: the compiler's own fence for a barrier would
// otherwise be merged into the wait and turn it into vmcnt(0).  The memory
// clobber keeps LDS accesses on their side of the barrier.
template <int VM>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(VM) : "memory");
}

// One workgroup: 8 waves of 32 (row, head) pairs each, two waves per SIMD.
// Per 32-key sub-block and wave: 8 MFMAs of Q K^T, 8 of P V, 17
// exponentials and about 65 other VALU operations.
template <bool WITH_O>
__global__ __launch_bounds__(512, 1) void attn_fwd(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_index,
    const int32_t* __restrict__ rows, sx_layout lay, int n_pages,
    const uint16_t* __restrict__ kpool, const uint16_t* __restrict__ vpool, int hkv, int G,
    uint16_t* __restrict__ o, float* __restrict__ lse, const AttnItem* __restrict__ items,
    const int32_t* __restrict__ counters, float* __restrict__ part_ml,
    uint16_t* __restrict__ part_o, int max_slots, float scale_log2) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Stage* st = reinterpret_cast<Stage*>(smem_raw);

  const int g = blockIdx.x % hkv;
  const int ii = blockIdx.x / hkv;
  if (ii >= counters[0] || n_pages <= 0 || lay.max_pages <= 0) return;
  const AttnItem it = items[ii];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hl = lane >> 5;
  const int hq = G * hkv;
  const int req = it.req;
  const int seq0 = lay.seq_start[req];
  const int seq_len = lay.seq_start[req + 1] - seq0;
  const int k0 = it.k0;
  const int k1 = min(it.k1, seq_len);
  if (k1 <= k0) return;

  // ---- this lane's (row, head) pair: query operand and position -------------
  constexpr int NT = 512;                  // threads per workgroup
  const int npairs = it.nrows * G;
  const int pair = 32 * w + (lane & 31);
  int pos_q;
  const uint16_t* qptr;
  {
    const bool valid = pair < npairs;
    const int r = pair / G, hh = pair - r * G;
    const int m = it.row0 + (valid ? r : 0);
    const int row_tok = rows ? rows[m] : m;
    // Causal limit, clamped to the item's last key: the sub-blocks the
    // pipeline runs past the item's end are then masked for every pair.
    pos_q = valid ? min(row_tok - seq0, k1 - 1) : k1 - 1;
    // (A pair past the tile reads a valid row's Q; its results are never
    // stored.)
    qptr = q + ((size_t)(q_index ? q_index[m] : m) * hq + g * G + hh) * 128 + hl * 8;
  }
  int wave_pmin = pos_q;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wave_pmin = min(wave_pmin, __shfl_xor(wave_pmin, off));

  // ---- K/V stages: global -> LDS directly (global_load_lds_dwordx4) ---------
  // A wave instruction writes 64 x 16 B = 1 KB of LDS, lane L at byte 16 L.
  // Each wave copies half a page of each 64-key block (K rows 8w .. 8w+7,
  // and the matching 64 head dimensions of its V page-head), 2 KB of K and
  // 2 KB of V, so page ids are wave-uniform and per-lane offsets constants.
  // K stage: 64 key rows x 256 B; row R keeps 16-byte chunk c at slot
  //   c ^ (R & 15) (16 rows read together hit 16 distinct bank groups).
  // V stage: the page layout itself, [4 pages][128 d][16 keys]; row d keeps
  //   its two 16-byte halves (keys 0-7, 8-15) swapped when (d >> 3) is odd.
  // Pages past the item's last key are replaced by its last page (finite
  // data, masked or zeroed); an invalid page id reads page 0.
  const int32_t* bt = lay.block_table + (size_t)req * lay.max_pages;
  const int kmax = k1 - 1;                 // last key of this item
  const int last_pi = max(min(kmax / kPage, lay.max_pages - 1), 0);
  constexpr int NCP = 2;                   // copies of 1 KB per wave for K (and for V)
  const int wpart = w & 1;                 // which half of its page a wave copies
  uint32_t koff[NCP], voff[NCP];           // byte offsets inside a page-head
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int slot = 8 * wpart + 4 * i + (lane >> 4);            // key row inside the page
    koff[i] = (uint32_t)(slot * 128 + (((lane & 15) ^ slot) * 8)) * 2u;
    const int d = 64 * wpart + 32 * i + (lane >> 1);
    voff[i] = (uint32_t)(d * 16 + (((lane & 1) ^ ((d >> 3) & 1)) * 8)) * 2u;
  }
  const size_t head_bytes = (size_t)kPage * 128 * 2;      // one page-head, 4 KB
  // Page id of this wave's page of the block at kb (scalar load: the wave
  // index is made wave-uniform).  Fetched one stage ahead of its use, so the
  // load latency is not paid when the copies are issued.
  // The block table is read-only for the whole kernel, so it is read through
  // the constant address space: a scalar load (s_load, counted by lgkmcnt)
  // rather than a vector load whose vmcnt wait would also wait for the
  // stage copies in flight.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  typedef __attribute__((address_space(4))) const int32_t* cptr_t;
  const cptr_t btc = (cptr_t)bt;
  const int wpage = wu >> 1;                // this wave's page of a block
  auto page_of_block = [&](int kb) __attribute__((always_inline)) {
    const int pi = min(kb / kPage + wpage, last_pi);
    const int pg = btc[pi];
    return (pg >= 0 && pg < n_pages) ? pg : 0;
  };
  // The K and V halves of a stage are issued separately (at different points
  // of an iteration) so that a wave never queues all its copies at once.
  auto issue_k = [&](int pg, int s) __attribute__((always_inline)) {
    const size_t base = ((size_t)pg * hkv + g) * head_bytes;
    const unsigned char* kp = reinterpret_cast<const unsigned char*>(kpool) + base;
    unsigned char* kst = reinterpret_cast<unsigned char*>(&st[s].k[8 * wu][0]);
#pragma unroll
    for (int i = 0; i < NCP; ++i)
      copy16_to_lds(kp + koff[i], kst + i * 1024);
  };
  auto issue_v = [&](int pg, int s) __attribute__((always_inline)) {
    if (!WITH_O) return;
    const size_t base = ((size_t)pg * hkv + g) * head_bytes;
    const unsigned char* vp = reinterpret_cast<const unsigned char*>(vpool) + base;
    unsigned char* vst = reinterpret_cast<unsigned char*>(&st[s].v[wpage][64 * (wu & 1)][0]);
#pragma unroll
    for (int i = 0; i < NCP; ++i)
      copy16_to_lds(vp + voff[i], vst + i * 1024);
  };
  auto issue_stage = [&](int pg, int s) __attribute__((always_inline)) {
    issue_k(pg, s);
    issue_v(pg, s);
  };
  // Zero the values of keys past kmax in a resident stage (P is 0 there, but
  // those slots may hold anything, and 0 * NaN would poison O).
  auto zero_tail = [&](int kb, int s) __attribute__((always_inline)) {
    const int first = kmax + 1 - kb;       // first key offset to clear
    if (!WITH_O || first >= KB) return;
    uint16_t* vs = &st[s].v[0][0][0];
    for (int u = tid; u < 128 * KB; u += NT) {
      const int key = u & (KB - 1), d = u >> 6;
      if (key < first) continue;
      const int j = key >> 4, kk = key & 15;
      const int half = (kk >> 3) ^ ((d >> 3) & 1);
      vs[(j * 128 + d) * kPage + half * 8 + (kk & 7)] = 0;
    }
  };
  // After the stage barrier: waits for the scalar page-id load (and the LDS
  // reads still in flight, which lgkmcnt counts with it), as a real
  // s_waitcnt the compiler's wait insertion sees.  With a scalar load
  // pending, scalar results may return out of order with LDS reads, so
  // every later wait for an LDS read would have to be lgkmcnt(0) and drain
  // all of the step's LDS reads in flight.
  auto lgkm_settled = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7, lgkmcnt 0 (gfx9 encoding)
  };
  // Workgroup barrier after this wave's LDS writes, leaving the stage copies
  // in flight.
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // K row read by this lane for the S^T A operand: inside a 32-key sub-block
  // the MFMA row mrow holds key kperm(mrow), so that accumulator register v
  // of lane half hl holds key 16*(v>>3) + 8*hl + (v&7) of the sub-block.
  const int mrow = lane & 31;
  const int kperm = 16 * (mrow >> 4) + 8 * ((mrow >> 2) & 1) + 4 * ((mrow >> 3) & 1) + (mrow & 3);

  // K operand of sub-block h (keys 32h .. 32h+31) of stage s: 8 x 16 B.
  auto load_k = [&](int s, int h, bf16x8 (&kf)[8]) __attribute__((always_inline)) {
    const int R = h * 32 + kperm;
    const uint16_t* kr = &st[s].k[R][0];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int slot = (2 * kk + hl) ^ (R & 15);
      kf[kk] = *reinterpret_cast<const bf16x8*>(kr + slot * 8);
    }
  };
  // V^T operand of sub-block h of stage s: 8 x 16 B.
  auto load_v = [&](int s, int h, bf16x8 (&vf)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int md = 0; md < 4; ++md) {
        const int d = md * 32 + (lane & 31);
        const int half = hl ^ ((d >> 3) & 1);
        vf[ks * 4 + md] = *reinterpret_cast<const bf16x8*>(&st[s].v[2 * h + ks][d][half * 8]);
      }
  };

  bf16x8 qf[8];                            // Q^T operand, 32 pairs x 128 d
  f32x16 oacc[4];                          // O^T, 128 d x 32 pairs
#pragma unroll
  for (int md = 0; md < 4; ++md) oacc[md] = f32x16{};
  bf16x8 vf[8];                            // V^T operand of the next P V
  float m_run = -INFINITY, alpha = 1.f;    // running max (raw logit units), O scale
  // Running row sums as four partial sums (short add chains); the first add
  // of each chain is an fma with alpha, which rescales them.
  float lp[4] = {0.f, 0.f, 0.f, 0.f};
  const float c = scale_log2;

  // S^T of a sub-block: 8 MFMAs, one dependent chain (gfx950 runs a chain
  // on one accumulator faster than MFMAs alternating between accumulators).
  auto qk = [&](const bf16x8 (&kf)[8], f32x16& S) __attribute__((always_inline)) {
    S = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], S, 0, 0, 0);
  };
  // O^T += V^T . P^T for one sub-block: 8 MFMAs, two in a row on each
  // accumulator.
  auto pv = [&](const bf16x8 (&P)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks * 4 + md], P[ks], oacc[md], 0, 0, 0);
  };

  // Softmax of a sub-block (keys kb .. kb+31): S -> P (bf16, B operand of
  // PV).  The running max is raised only when the sub-block exceeds it by
  // more than 2^8 in the exp2 domain (alpha is then the O scale factor).
  // Returns true if O must be rescaled.
  auto softmax = [&](f32x16& S, bool mask, int kb, bf16x8 (&P)[2]) __attribute__((always_inline)) {
    if (mask) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb + 16 * (v >> 3) + 8 * hl + (v & 7);
        S[v] = key > pos_q ? -INFINITY : S[v];
      }
    }
    // tree of 3-input maxima (8 v_max3, depth 3)
    float t[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) t[i] = fmaxf(fmaxf(S[3 * i], S[3 * i + 1]), S[3 * i + 2]);
    const float u0 = fmaxf(fmaxf(t[0], t[1]), t[2]);
    const float u1 = fmaxf(fmaxf(t[3], t[4]), S[15]);
    const float mx = half_max(fmaxf(u0, u1));
    const bool any = __ballot((mx - m_run) * c > 8.f) != 0ull;
    const float m_new = any ? fmaxf(m_run, mx) : m_run;
    // A key chunk of a split tile can lie wholly past a row's position: the
    // row then has no key yet, m stays -inf, and the exponent reference is 0
    // (p = 0, alpha = 0) instead of -inf - -inf.  Only masked steps can see
    // such a row.
    const float m_ref = (mask && m_new == -INFINITY) ? 0.f : m_new;
    alpha = __builtin_amdgcn_exp2f((m_run - m_ref) * c);
    m_run = m_new;
    const float mc = m_ref * c;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pv_[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv_[i] = __builtin_amdgcn_exp2f(fmaf(S[ks * 8 + i], c, -mc));
        lp[i & 3] = (ks == 0 && i < 4) ? fmaf(lp[i & 3], alpha, pv_[i]) : lp[i & 3] + pv_[i];
      }
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = pack_bf2(pv_[2 * i], pv_[2 * i + 1]);
      P[ks] = __builtin_bit_cast(bf16x8, pk);
    }
    return any;
  };
  // O *= alpha.  The empty volatile asm keeps this a real (rarely taken)
  // branch: the compiler would otherwise speculate the 64 multiplies into
  // every step.
  auto rescale = [&]() __attribute__((always_inline)) {
    asm volatile("");
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[md][v] *= alpha;
  };

  // One step j of a three-stage pipeline over 32-key sub-blocks: P V of
  // sub-block j (vf, P; the V^T operand was read in the previous step), Q K^T
  // of sub-block j+2 (into Sn, K read from LDS in this step), the V^T operand
  // of sub-block j+1 for the next step, and the softmax of sub-block j+1
  // (Sc -> Pn).  O is rescaled at the end of the step (after P V j, before
  // P V j+1) if the softmax raised the running max.
  // Sub-block x lives in ring slot (x / 2) % NSTAGE, half x % 2.
  auto step = [&](auto mask_tag, int j, f32x16& Sc, f32x16& Sn, const bf16x8 (&P)[2],
                  bf16x8 (&Pn)[2]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (WITH_O) pv(P);
    bf16x8 kf[8];
    load_k(((j + 2) >> 1) % NSTAGE, j & 1, kf);
    qk(kf, Sn);
    if (WITH_O) load_v(((j + 1) >> 1) % NSTAGE, (j + 1) & 1, vf);
    const bool r = softmax(Sc, MASK, k0 + 32 * (j + 1), Pn);
    // The softmax results are used only in the next step; pinned here, they
    // stay in this step's scheduling region instead of sinking below the
    // rescale branch.
    asm volatile("" : "+v"(Pn[0]), "+v"(Pn[1]));
    asm volatile("" : "+v"(lp[0]), "+v"(lp[1]), "+v"(lp[2]), "+v"(lp[3]));
    if (WITH_O && r) rescale();
  };

  const int n_sub = (k1 - k0 + 31) / 32;
  const int n_stage = (n_sub + 1) / 2;
  const bool tail_partial = k0 + n_stage * KB - 1 > kmax;   // last stage holds keys past kmax
  // Stage copies: stages 0-2 in the prologue, then one per iteration (stage
  // b+3 at the start of iteration b, into the slot of stage b-1, which no
  // wave reads after the barrier there).  Past the item's end the copies
  // repeat its last page into slots no one reads any more, so the copy count
  // per iteration is fixed and each wait is a constant: all but the newest
  // stage's copies complete.
  constexpr int per_stage = WITH_O ? 2 * NCP : NCP;   // copies per wave per stage
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i) issue_stage(page_of_block(k0 + i * KB), i);
  // Q is loaded after the first stage copies are on their way (one wait
  // covers both).
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qptr + kk * 16));
  vm_wait_barrier<(NSTAGE - 2) * per_stage>();   // stage 0 resident
  lgkm_settled();
  if (tail_partial && n_stage == 1) {
    zero_tail(k0, 0);
    lds_barrier();
  }
  // prologue: S of sub-blocks 0 (even) and 1 (odd), softmax of sub-block 0,
  // V operand of sub-block 0
  f32x16 S_even, S_odd;
  bf16x8 Pa[2], Pb[2];
  {
    bf16x8 kf[8];
    load_k(0, 0, kf);
    qk(kf, S_even);
    load_k(0, 1, kf);
    qk(kf, S_odd);
    softmax(S_even, k0 + 31 > wave_pmin, k0, Pa);   // O is still 0: no rescale
    if (WITH_O) load_v(0, 0, vf);
  }

  // Iteration b = steps 2b (A) and 2b+1 (B), after a barrier that makes
  // stage b+1 resident and frees the slot of stage b-1:
  //   step A: PV 2b (stage b), QK^T 2b+2 (stage b+1), V of 2b+1, softmax 2b+1
  //   step B: PV 2b+1 (stage b), QK^T 2b+3 (stage b+1), V of 2b+2, softmax 2b+2
  // The K half of stage b+3 is copied before step A, its V half before
  // step B.  Work past the item's last sub-block is harmless (QK^T results
  // unused, softmax fully masked since causal limits are clamped to the
  // item's last key, reads inside the ring) except PV, so the loop exits
  // right after the last PV.  Sub-blocks wholly below the tile's first query
  // row need no causal mask: iterations b < b_plain are unmasked (and never
  // reach the exit).  The last stage's values past the item's end are
  // zeroed once it is resident; its V is first read in step B, after a
  // barrier that orders those writes.
  const int tile_pmin = it.pad0;
  const int n_plain_sub = max(0, (min(tile_pmin, kmax) - k0 + 1) / 32);
  const int b_plain = max(0, (n_plain_sub - 1) / 2);
  // The page id of stage b+3 is loaded (scalar) just before the barrier of
  // iteration b, whose wait covers its latency.
  int pg_next = 0;
  auto barrier_copy_k = [&](int b) __attribute__((always_inline)) {
    pg_next = page_of_block(k0 + (b + 3) * KB);
    vm_wait_barrier<per_stage>();             // stage b+1 resident, b+2 may be in flight
    lgkm_settled();
    if (tail_partial && b + 1 == n_stage - 1) {
      zero_tail(k0 + (b + 1) * KB, (b + 1) % NSTAGE);
      lds_barrier();
    }
    issue_k(pg_next, (b + 3) % NSTAGE);
  };
  auto copy_v = [&](int b) __attribute__((always_inline)) {
    issue_v(pg_next, (b + 3) % NSTAGE);
  };
  int b = 0;
  for (; b < b_plain; ++b) {
    barrier_copy_k(b);
    step(std::false_type{}, 2 * b, S_odd, S_even, Pa, Pb);
    copy_v(b);
    step(std::false_type{}, 2 * b + 1, S_even, S_odd, Pb, Pa);
  }
  for (;; ++b) {
    barrier_copy_k(b);
    step(std::true_type{}, 2 * b, S_odd, S_even, Pa, Pb);
    if (2 * b + 1 >= n_sub) break;
    copy_v(b);
    step(std::true_type{}, 2 * b + 1, S_even, S_odd, Pb, Pa);
    if (2 * b + 2 >= n_sub) break;
  }
  // No stage copy may still be writing LDS when the workgroup ends.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue ----------------------------------------------------------------
  // Final outputs go through LDS (the stage ring is free once every wave's
  // copies have landed): each wave writes its 32 normalised bf16 output rows
  // of 256 bytes there, then stores whole rows, 16 lanes per row, so HBM sees
  // full lines instead of 8-byte pieces of 32 rows per instruction.  Rows are
  // padded to 272 bytes so the row-strided writes spread over the banks.
  constexpr int kStgLd = 136;
  static_assert(8 * 32 * kStgLd * 2 <= NSTAGE * (int)sizeof(Stage), "output staging fits the ring");
  const bool final_out = it.slot < 0;
  uint16_t* stg = reinterpret_cast<uint16_t*>(smem_raw) + (size_t)w * 32 * kStgLd;
  if (WITH_O && final_out) __syncthreads();
  const bool valid = pair < npairs;
  const int r = pair / G, hh = pair - r * G;
  const int m = it.row0 + r;
  const int h = g * G + hh;
  const float l_tot = half_sum((lp[0] + lp[1]) + (lp[2] + lp[3]));
  const float m2 = m_run * c;                         // log2-domain max
  if (final_out) {
    if (lse && valid && hl == 0) lse[(size_t)m * hq + h] = (m2 + __log2f(l_tot)) * kLn2;
    if (WITH_O) {
      const float inv = 1.f / l_tot;
      uint16_t* sp = stg + (lane & 31) * kStgLd + 4 * hl;
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 pk;
          pk[0] = pack_bf2(oacc[md][4 * j] * inv, oacc[md][4 * j + 1] * inv);
          pk[1] = pack_bf2(oacc[md][4 * j + 2] * inv, oacc[md][4 * j + 3] * inv);
          *reinterpret_cast<u32x2*>(sp + md * 32 + 8 * j) = pk;
        }
    }
  } else if (it.slot < max_slots) {
    // Split tile: the chunk's max, row sum and normalised output go to the
    // partial slot.  The output is stored as fp16 scaled by 2^-e, with e the
    // smallest power that brings the pair's largest |o| below 2^15 (0 for
    // |o| < 2^15), so any value bf16 can hold survives; the merge multiplies
    // by 2^e again.
    const size_t pslot = ((size_t)it.slot * hkv + g) * PAIRS + pair;
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;   // a chunk past the row: o = 0
    float scl = 1.f;
    if (WITH_O) {
      float amax = 0.f;
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(oacc[md][v]));
      amax = half_max(amax) * inv;
      if (amax >= 32768.f && amax <= 3.0e38f) {
        const int e = __builtin_amdgcn_frexp_expf(amax);       // amax = f 2^e, f in [0.5, 1)
        scl = __builtin_ldexpf(1.f, e - 15);
        inv = __builtin_ldexpf(inv, 15 - e);
      }
    }
    if (hl == 0) {
      part_ml[4 * pslot] = m2;
      part_ml[4 * pslot + 1] = l_tot;
      part_ml[4 * pslot + 2] = scl;
    }
    if (WITH_O) {
      uint16_t* op = part_o + pslot * 128 + 4 * hl;
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 pk;
          pk[0] = pack_h2(oacc[md][4 * j] * inv, oacc[md][4 * j + 1] * inv);
          pk[1] = pack_h2(oacc[md][4 * j + 2] * inv, oacc[md][4 * j + 3] * inv);
          *reinterpret_cast<u32x2*>(op + md * 32 + 8 * j) = pk;
        }
    }
  }
  if (WITH_O && final_out) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's staging writes are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pl = 4 * i + (lane >> 4), ch = lane & 15;
      const int pp = 32 * w + pl;
      if (pp < npairs) {
        const int rr = pp / G, hh2 = pp - rr * G;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + pl * kStgLd + ch * 8);
        *reinterpret_cast<u32x4*>(o + ((size_t)(it.row0 + rr) * hq + g * G + hh2) * 128 + ch * 8) = v;
      }
    }
  }
}

// Combines the key chunks of split tiles (chunk order fixed):
//   M = max_c m_c,  w_c = l_c 2^(m_c - M),  O = sum_c w_c O_c / sum_c w_c,
//   LSE = (M + log2 sum_c w_c) ln 2.
// One workgroup per (merge tile, kv head, group of 16 pairs); 16 threads per
// pair, 8 head dimensions per thread.  Partial outputs are normalised fp16
// values times 2^-e; the slot's third float holds 2^e.
constexpr int kMergePairs = 16;
template <bool WITH_O>
__global__ __launch_bounds__(256) void attn_merge(
    const MergeTile* __restrict__ merges, const int32_t* __restrict__ counters, int hkv, int G,
    const float* __restrict__ part_ml, const uint16_t* __restrict__ part_o,
    uint16_t* __restrict__ o, float* __restrict__ lse, int max_slots) {
  const int grp = blockIdx.x % (PAIRS / kMergePairs);
  const int g = (blockIdx.x / (PAIRS / kMergePairs)) % hkv;
  const int mi = blockIdx.x / (PAIRS / kMergePairs) / hkv;
  if (mi >= counters[1]) return;
  const MergeTile mt = merges[mi];
  if (mt.slot0 < 0 || mt.slot0 + mt.n_chunks > max_slots) return;
  const int hq = G * hkv;
  const int npairs = mt.nrows * G;
  const int sub = threadIdx.x & 15;
  const int p = grp * kMergePairs + (threadIdx.x >> 4);
  if (p < npairs) {
    float M = -INFINITY;
    for (int c = 0; c < mt.n_chunks; ++c) {
      const size_t ps = ((size_t)(mt.slot0 + c) * hkv + g) * PAIRS + p;
      M = fmaxf(M, part_ml[4 * ps]);
    }
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float wsum = 0.f;
    for (int c = 0; c < mt.n_chunks; ++c) {
      const size_t ps = ((size_t)(mt.slot0 + c) * hkv + g) * PAIRS + p;
      const float wc = part_ml[4 * ps + 1] * __builtin_amdgcn_exp2f(part_ml[4 * ps] - M);
      wsum += wc;
      if (WITH_O) {
        const float wo = wc * part_ml[4 * ps + 2];
        const u32x4 raw = *reinterpret_cast<const u32x4*>(part_o + ps * 128 + sub * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2_t a = unpack_h2(raw[e]);
          acc[2 * e] = fmaf(wo, a[0], acc[2 * e]);
          acc[2 * e + 1] = fmaf(wo, a[1], acc[2 * e + 1]);
        }
      }
    }
    const int r = p / G, hh = p - r * G;
    const int m = mt.row0 + r;
    const int h = g * G + hh;
    if (lse && sub == 0) lse[(size_t)m * hq + h] = (M + __log2f(wsum)) * kLn2;
    if (WITH_O) {
      const float inv = 1.f / wsum;
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = pack_bf2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
      *reinterpret_cast<u32x4*>(o + ((size_t)m * hq + h) * 128 + sub * 8) = pk;
    }
  }
}

// fp32 storage: one wave per (row, query head); lanes split the head
// dimension, keys are visited in order with an online softmax.
template <int D>
__global__ __launch_bounds__(64) void attn_rows_f32(
    const float* __restrict__ q, const int32_t* __restrict__ q_index,
    const int32_t* __restrict__ rows, int n_rows, sx_layout lay, int n_pages,
    const float* __restrict__ kpool, const float* __restrict__ vpool, int hkv, int hq,
    float* __restrict__ o, float* __restrict__ lse, float scale) {
  constexpr int E = D / 64;
  const int m = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int g = h / (hq / hkv);
  const int tok = rows ? rows[m] : m;
  const int r = find_request(lay.seq_start, lay.n_req, tok);
  if (r < 0) return;
  const int i = tok - lay.seq_start[r];
  const float* qp = q + ((size_t)(q_index ? q_index[m] : m) * hq + h) * D;
  float qv[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = qp[lane + 64 * e];
    acc[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int j = 0; j <= i; ++j) {
    const int page = page_of(lay, n_pages, r, j);
    if (page < 0) continue;
    const float* kp = kpool + (((size_t)page * hkv + g) * kPage + (j & (kPage - 1))) * D;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part = fmaf(qv[e], kp[lane + 64 * e], part);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    const float sc = part * scale;
    const float m_new = fmaxf(m_run, sc);
    const float alpha = expf(m_run - m_new);
    const float p = expf(sc - m_new);
    l_run = l_run * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float vv = vpool[(((size_t)page * hkv + g) * D + lane + 64 * e) * kPage + (j & (kPage - 1))];
      acc[e] = acc[e] * alpha + p * vv;
    }
    m_run = m_new;
  }
  if (o) {
#pragma unroll
    for (int e = 0; e < E; ++e) o[((size_t)m * hq + h) * D + lane + 64 * e] = acc[e] / l_run;
  }
  if (lse && lane == 0) lse[(size_t)m * hq + h] = m_run + logf(l_run);
}

// Whether a work list over n_rows rows can hold split tiles.  Every
// request's rows are tiled separately, so there are at least n_rows / M
// tiles: with n_rows >= M * target no tile is split (the work list is told
// so) and the merge pass is not launched.
bool attn_may_split(int n_rows, int G, int hkv) {
  return (long long)n_rows < (long long)rows_per_tile(G) * items_per_head(hkv);
}

// The work list (tiles, items, merges, counters) into ws.  Its offsets in
// ws do not depend on whether outputs are produced.
sx_status plan_bf16(const sx_dims& dims, const sx_layout& lay, const int32_t* rows,
                    const int32_t* row_start, int n_rows, void* ws, hipStream_t stream) {
  const int hq = dims.n_q_heads, hkv = dims.n_kv_heads, G = hq / hkv;
  const WsLayout L = ws_layout(n_rows, lay.n_req, G, hkv, true);
  char* base = static_cast<char*>(ws);
  build_work<<<1, kBuildThreads, (size_t)(lay.n_req + 1) * sizeof(int), stream>>>(
      row_start, rows, lay.seq_start, lay.n_req, n_rows, rows_per_tile(G), items_per_head(hkv),
      L.max_tiles, L.max_items, attn_may_split(n_rows, G, hkv) ? 1 : 0,
      reinterpret_cast<TileInfo*>(base + L.tiles), reinterpret_cast<AttnItem*>(base + L.items),
      reinterpret_cast<MergeTile*>(base + L.merges), reinterpret_cast<int32_t*>(base + L.counters));
  return check_launch("attention work list");
}

// Attention and merge over the work list already in ws.
template <bool WITH_O>
sx_status run_bf16(const sx_dims& dims, const sx_layout& lay, const void* q,
                   const int32_t* q_index, const int32_t* rows, int n_rows, const sx_pages& kv,
                   void* o, float* lse, void* ws, hipStream_t stream) {
  const int hq = dims.n_q_heads, hkv = dims.n_kv_heads, G = hq / hkv;
  const WsLayout L = ws_layout(n_rows, lay.n_req, G, hkv, WITH_O);
  char* base = static_cast<char*>(ws);
  int32_t* counters = reinterpret_cast<int32_t*>(base + L.counters);
  AttnItem* items = reinterpret_cast<AttnItem*>(base + L.items);
  MergeTile* merges = reinterpret_cast<MergeTile*>(base + L.merges);
  float* part_ml = reinterpret_cast<float*>(base + L.part_ml);
  uint16_t* part_o = WITH_O ? reinterpret_cast<uint16_t*>(base + L.part_o) : nullptr;
  const size_t smem = NSTAGE * sizeof(Stage);
  sx_status st = allow_lds((const void*)attn_fwd<WITH_O>, smem, "attention");
  if (st != SX_OK) return st;
  const float scale_log2 = kLog2e / sqrtf((float)dims.head_dim);
  attn_fwd<WITH_O><<<L.max_items * hkv, 512, smem, stream>>>(
      (const uint16_t*)q, q_index, rows, lay, kv.n_pages, (const uint16_t*)kv.k,
      (const uint16_t*)kv.v, hkv, G, (uint16_t*)o, lse, items, counters, part_ml, part_o,
      L.max_items, scale_log2);
  st = check_launch("attention");
  if (st != SX_OK) return st;
  if (!attn_may_split(n_rows, G, hkv)) return SX_OK;
  attn_merge<WITH_O><<<L.max_tiles * hkv * (PAIRS / kMergePairs), 256, 0, stream>>>(merges, counters, hkv, G, part_ml,
                                                           part_o, (uint16_t*)o, lse, L.max_items);
  return check_launch("attention merge");
}

sx_status run_f32(const sx_dims& dims, const sx_layout& lay, const void* q, const int32_t* q_index,
                  const int32_t* rows, int n_rows, const sx_pages& kv, void* o, float* lse,
                  hipStream_t stream) {
  const int hq = dims.n_q_heads, hkv = dims.n_kv_heads, d = dims.head_dim;
  const float scale = 1.f / sqrtf((float)d);
  dim3 grid(n_rows, hq);
  if (d == 64)
    attn_rows_f32<64><<<grid, 64, 0, stream>>>((const float*)q, q_index, rows, n_rows, lay,
                                               kv.n_pages, (const float*)kv.k, (const float*)kv.v,
                                               hkv, hq, (float*)o, lse, scale);
  else
    attn_rows_f32<128><<<grid, 64, 0, stream>>>((const float*)q, q_index, rows, n_rows, lay,
                                                kv.n_pages, (const float*)kv.k, (const float*)kv.v,
                                                hkv, hq, (float*)o, lse, scale);
  return check_launch("attention (fp32)");
}

}  // namespace

size_t attn_ws_bytes(const sx_dims& dims, int n_rows, int n_req, bool with_o) {
  if (dims.dtype != SX_BF16 || n_rows <= 0) return 0;
  const int G = dims.n_q_heads / dims.n_kv_heads;
  return ws_layout(n_rows, n_req, G, dims.n_kv_heads, with_o).total;
}

sx_status launch_attention_plan(const sx_dims& dims, const sx_layout& lay, const int32_t* rows,
                                const int32_t* row_start, int n_rows, void* ws, hipStream_t stream) {
  if (n_rows == 0 || dims.dtype != SX_BF16) return SX_OK;   // fp32 rows need no work list
  return plan_bf16(dims, lay, rows, row_start, n_rows, ws, stream);
}

sx_status launch_attention_run(const sx_dims& dims, const sx_layout& lay, const void* q,
                               const int32_t* q_index, const int32_t* rows, int n_rows,
                               const sx_pages& kv, void* o, float* lse, void* ws,
                               hipStream_t stream) {
  if (n_rows == 0) return SX_OK;
  if (dims.dtype != SX_BF16) return run_f32(dims, lay, q, q_index, rows, n_rows, kv, o, lse, stream);
  return o ? run_bf16<true>(dims, lay, q, q_index, rows, n_rows, kv, o, lse, ws, stream)
           : run_bf16<false>(dims, lay, q, q_index, rows, n_rows, kv, o, lse, ws, stream);
}

sx_status launch_attention(const sx_dims& dims, const sx_layout& lay, const void* q,
                           const int32_t* q_index, const int32_t* rows,
                           const int32_t* row_start, int n_rows, const sx_pages& kv, void* o,
                           float* lse, void* ws, hipStream_t stream) {
  const sx_status st = launch_attention_plan(dims, lay, rows, row_start, n_rows, ws, stream);
  if (st != SX_OK) return st;
  return launch_attention_run(dims, lay, q, q_index, rows, n_rows, kv, o, lse, ws, stream);
}

}  // namespace sx
