// Sparse-KV recomputation (SparseX paper §3.4: K/V of the Sparse-Q rows and
// the selected top-k rows are recomputed in the same forward pass; §4.5:
// recomputed tokens take the normal attention path).
//
//   [q | k | v] = x[rows] . W_qkv^T ;  q, k rotated by R_pos ;
//   k, v scattered into the request's pages, q written densely.
//
// bf16 path: MFMA GEMM (v_mfma_f32_32x32x16_bf16), 256x128, 256x256 or
// 256x384 output tiles (one, two or three whole heads of 128, so both halves
// of every rotate-half pair are in the tile).  Tiles are assigned XCD-contiguously (workgroup b
// runs on XCD b % 8) and grouped 4 row-tiles at a time so that concurrently
// running workgroups share W and X slices in their XCD's L2.  The epilogue
// stages the fp32 tile in LDS, applies RoPE with the fp64-built table,
// rounds to bf16 and writes 16-byte chunks (Q, K) or page columns (V).
#include <type_traits>

#include "realign_job.hpp"
#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

namespace {

constexpr int BN = 128, BK = 64;
constexpr int LDC = BN + 4;          // padded fp32 row of the staged output tile
constexpr int GROUP_M = 4;

// bf16 GEMM, 256-row output tiles of one, two or three heads.  K-steps of
// 64 go global -> LDS directly (global_load_lds_dwordx4, copy16_to_lds) into
// a ring of stages;
// each 128-byte LDS row keeps its 16-byte chunk c at position c ^ (row & 7),
// so the rows an MFMA operand read touches spread over the banks.  Eight
// waves, two per SIMD, each of 64 columns and 64 or 128 rows in 32 x 32
// MFMA tiles (one wave's barrier and LDS waits overlap the other's MFMAs;
// for one head, four waves of 128 x 64 were 7% slower than eight of
// 64 x 64); the operands of k-slice ks+1 are read from LDS while the MFMAs
// of slice ks run.
constexpr int BM2 = 256;
constexpr int GW = 8;                  // waves per workgroup: two per SIMD
constexpr int GT = 64 * GW;            // threads per workgroup
constexpr int NCA = BM2 * BK * 2 / 1024 / GW;   // 1 KB stage copies per wave: A
// HPT heads (128 columns each) per tile.  HPT = 1: 48 KB stages in a ring
// of 3, waves 4 x 2 of 64 x 64.  HPT = 2 (256 x 256 tiles, 1.5x the flops
// per staged byte): 64 KB stages in a ring of 2, waves 2 x 4 of 128 x 64.
// HPT = 3 (256 x 384 tiles, 1.8x): 80 KB stages in a ring of 2 (the whole
// LDS), waves 4 x 2 of 64 x 192 (192 accumulator registers per lane, so only
// the next B fragment is read ahead, not the next k-slice's operands).
template <int HPT>
struct GemmCfg {
  static constexpr int BNT = BN * HPT;              // output columns per tile
  static constexpr int NST = HPT == 1 ? 3 : 2;      // ring stages
  static constexpr int WGN = HPT == 2 ? 4 : 2;      // waves along N
  static constexpr int WGM = GW / WGN;              // waves along M
  static constexpr int WROWS = BM2 / WGM;           // output rows per wave
  static constexpr int WCOLS = BNT / WGN;           // output columns per wave
  static constexpr int MI = WROWS / 32;             // 32 x 32 MFMA tiles per wave along M
  static constexpr int NJ = WCOLS / 32;             // ... and along N
  static constexpr int NBUF = HPT == 3 ? 1 : 2;     // k-slices of operands in registers
  static constexpr int NCB = BNT * BK * 2 / 1024 / GW;   // 1 KB stage copies per wave: B
};
template <int HPT>
struct Gemm2Stage {
  uint16_t a[BM2][BK];
  uint16_t b[BN * HPT][BK];
};
// The epilogue's view of the LDS, once the ring is no longer needed: one
// head of the output tile in fp32, and per output row the page of its token
// (-1 if the row or its page is invalid; for Q heads only row_ok matters),
// its slot and its RoPE position.
struct GemmEpi {
  float c[BM2][LDC];
  int32_t row_page[BM2];
  int32_t row_slot[BM2];
  int32_t row_pos[BM2];
  int32_t row_ok[BM2];
};
template <int HPT>
struct Gemm2Smem {
  union {
    Gemm2Stage<HPT> st[GemmCfg<HPT>::NST];
    GemmEpi epi;
  };
};

// Realign jobs of another layer's pool carried by a projection launch: the
// workgroups past the projection's tiles run them (launch_recompute_realign).
struct SideRealign {
  const uint16_t* ksrc;
  const uint16_t* vsrc;
  uint16_t* kdst;
  uint16_t* vdst;
  const sx_realign_job* jobs;
  int n_src_pages, n_dst_pages, n_jobs;
  int tile_blocks;             // blocks [0, tile_blocks) are projection tiles
};

template <int HPT>
__global__ __launch_bounds__(GT, 1) void qkv_gemm256_bf16(
    const uint16_t* __restrict__ x, int hidden, const int32_t* __restrict__ rows, int n_rows,
    const uint16_t* __restrict__ w, int head0, int n_tiles_m, int n_tiles_n, sx_layout lay,
    int n_pages, uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
    uint16_t* __restrict__ q_out, int hq, int hkv, SideRealign side) {
  using Cfg = GemmCfg<HPT>;
  constexpr int NST2 = Cfg::NST, WROWS = Cfg::WROWS, MI = Cfg::MI, NCB = Cfg::NCB;
  if ((int)blockIdx.x >= side.tile_blocks) {
    // a realign worker, on a compute unit the projection's tiles leave free:
    // an equal contiguous share of the side list, four pages at a time
    const int w = blockIdx.x - side.tile_blocks, nw = gridDim.x - side.tile_blocks;
    const int per = (side.n_jobs + nw - 1) / nw;
    realign_job_run<4, GT>(side.jobs, min(w * per, side.n_jobs), min((w + 1) * per, side.n_jobs),
                           side.ksrc, side.vsrc, side.kdst, side.vdst, side.n_src_pages,
                           side.n_dst_pages, hkv, lay.rope_tab, lay.rope_len, threadIdx.x);
    return;
  }
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Gemm2Smem<HPT>& sm = *reinterpret_cast<Gemm2Smem<HPT>*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;

  // ---- tile assignment: XCD-contiguous ranges, grouped along M ----------
  const int total = n_tiles_m * n_tiles_n;
  const int per_xcd = (total + 7) / 8;
  const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (t >= total) return;
  const int group = t / (GROUP_M * n_tiles_n);
  const int first_m = group * GROUP_M;
  const int gsz = min(n_tiles_m - first_m, GROUP_M);
  const int within = t % (GROUP_M * n_tiles_n);
  const int mt = first_m + within % gsz;
  const int nt = within / gsz;
  const int m0 = mt * BM2;
  const int head1 = head0 + HPT * nt;         // first head: 0..hq-1 Q, then K heads, then V heads
  const uint16_t* wt = w + (size_t)head1 * 128 * hidden;

  // ---- copy plan: lane L of copy i moves one 16-byte chunk --------------
  // A: rows 8*NCA*wave + 8*i + L/8 (i < NCA); B: rows 8*NCB*wave + 8*i + L/8
  // (i < NCB).
  // Row R's chunk c is stored at chunk position c ^ (R & 7) = L % 8, so the
  // lane loads chunk (L % 8) ^ (R & 7).  Rows past n_rows (or with a token
  // outside the sequence) read row 0 of x: finite data whose results are
  // never stored.
  size_t a_off[NCA];                         // byte offsets of this lane's chunks at k = 0
  uint32_t b_off[NCB];
#pragma unroll
  for (int i = 0; i < NCA; ++i) {
    const int R = 8 * NCA * wave + 8 * i + (lane >> 3);
    const int m = m0 + R;
    int tok = m < n_rows ? rows[m] : 0;
    if (tok < 0 || tok >= lay.n_tok) tok = 0;
    a_off[i] = ((size_t)tok * hidden + (size_t)(((lane & 7) ^ (R & 7)) * 8)) * 2u;
  }
#pragma unroll
  for (int i = 0; i < NCB; ++i) {
    const int R = 8 * NCB * wave + 8 * i + (lane >> 3);
    b_off[i] = ((uint32_t)R * (uint32_t)hidden + (uint32_t)(((lane & 7) ^ (R & 7)) * 8)) * 2u;
  }
  const unsigned char* xb = reinterpret_cast<const unsigned char*>(x);
  const unsigned char* wb = reinterpret_cast<const unsigned char*>(wt);
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const int n_k = hidden / BK;
  // Stage kt (k = 64 kt, clamped to the last step: the copies past the end
  // repeat it into a ring slot no one reads any more, keeping NCA + NCB
  // copies per wave and stage so each wait is a constant).
  auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)min(kt, n_k - 1) * BK * 2u;
    unsigned char* as = reinterpret_cast<unsigned char*>(&sm.st[slot].a[8 * NCA * wu][0]);
    unsigned char* bs = reinterpret_cast<unsigned char*>(&sm.st[slot].b[8 * NCB * wu][0]);
#pragma unroll
    for (int i = 0; i < NCA; ++i)
      copy16_to_lds(xb + a_off[i] + kb, as + i * 1024);
#pragma unroll
    for (int i = 0; i < NCB; ++i)
      copy16_to_lds(wb + b_off[i] + kb, bs + i * 1024);
  };

  constexpr int NJ = Cfg::NJ, NBUF = Cfg::NBUF;
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int s = 0; s < NST2 - 1; ++s) issue(s, s);
  for (int kt = 0; kt < n_k; ++kt) {
    const int slot = kt % NST2;
    // stage kt resident in every wave (the NST2 - 2 stages after it may be
    // in flight); the slot of stage kt-1 is free for stage kt+NST2-1
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((NST2 - 2) * (NCA + NCB)) : "memory");
    issue(kt + NST2 - 1, (kt + NST2 - 1) % NST2);
    const Gemm2Stage<HPT>& S = sm.st[slot];
    // With two operand buffers the operands of k-slice ks+1 are read while
    // the MFMAs of slice ks run.
    bf16x8 af[NBUF][MI], bfr[NBUF][NJ];
    auto load = [&](int ks, int buf) __attribute__((always_inline)) {
      const int ch = 2 * ks + lh;              // 16-byte chunk of this lane's k range
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int R = wm * WROWS + i * 32 + lr;
        af[buf][i] = *reinterpret_cast<const bf16x8*>(&S.a[R][(ch ^ (R & 7)) * 8]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int R = wn * Cfg::WCOLS + j * 32 + lr;
        bfr[buf][j] = *reinterpret_cast<const bf16x8*>(&S.b[R][(ch ^ (R & 7)) * 8]);
      }
    };
    if (NBUF == 2) {
      load(0, 0);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        if (ks + 1 < BK / 16) load(ks + 1, (ks + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);   // keep those reads ahead of this slice's MFMAs
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0, 0, 0);
      }
    } else {
      // one operand buffer (few operand registers live next to 192
      // accumulators): the A fragments of a slice, and the B fragments one
      // MFMA group ahead, so each B read has the previous group's MFMAs to
      // land behind (3% faster at 3,379 rows than reading each just before
      // its MFMAs)
      auto read_b = [&](int ks, int j) __attribute__((always_inline)) {
        const int R = wn * Cfg::WCOLS + j * 32 + lr;
        return *reinterpret_cast<const bf16x8*>(&S.b[R][((2 * ks + lh) ^ (R & 7)) * 8]);
      };
      bf16x8 b_next = read_b(0, 0);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = 2 * ks + lh;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int R = wm * WROWS + i * 32 + lr;
          af[0][i] = *reinterpret_cast<const bf16x8*>(&S.a[R][(ch ^ (R & 7)) * 8]);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bf16x8 bj = b_next;
          if (j + 1 < NJ) b_next = read_b(ks, j + 1);
          else if (ks + 1 < BK / 16) b_next = read_b(ks + 1, 0);
#pragma unroll
          for (int i = 0; i < MI; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0][i], bj, acc[i][j], 0, 0, 0);
        }
      }
    }
  }
  // all copies landed and every wave done with the ring before it becomes C
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  GemmEpi& ep = sm.epi;
  if (tid < BM2) {
    int r = -1, idx = 0;
    if (m0 + tid < n_rows) {
      const int tok = rows[m0 + tid];
      r = find_request(lay.seq_start, lay.n_req, tok);
      if (r >= 0) idx = tok - lay.seq_start[r];
    }
    ep.row_ok[tid] = r >= 0;
    ep.row_page[tid] = r >= 0 ? page_of(lay, n_pages, r, idx) : -1;
    ep.row_slot[tid] = idx & (kPage - 1);
    ep.row_pos[tid] = r >= 0 ? rope_pos(lay, r, idx) : 0;
  }

  // ---- epilogue, one head at a time: its fp32 columns -> LDS -------------
  // Each wave column (wn) runs its own copy of this code, so which
  // accumulators a wave still holds is known at compile time and a head's
  // accumulators are dead once staged.  With three heads the middle one,
  // split between the two wave columns, goes first: no wave then holds more
  // than two of its three heads' accumulators while the RoPE table entries
  // are in registers (in head order a wave held all of them and spilled).
  // Every copy passes the same barriers in the same order.
  auto store_head = [&](const int head) __attribute__((always_inline)) {
    if (head < hq + hkv) {
      // Q or K head: rotate-half pairs (e, e+64), 8 pairs per unit; a thread
      // takes 8 units (rows tid/8 + 32 k), first loading all their RoPE table
      // entries, then rotating and storing.
      const bool is_q = head < hq;
      const int g = head - hq;
      constexpr int kUnits = BM2 * 8 / GT;
      const int c = tid & 7;
      f32x4 tabv[kUnits][4];
#pragma unroll
      for (int k = 0; k < kUnits; ++k) {
        const int m = (tid >> 3) + (GT / 8) * k;
        const f32x4* tab = reinterpret_cast<const f32x4*>(lay.rope_tab + (size_t)ep.row_pos[m] * 128 + c * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) tabv[k][i] = tab[i];
      }
#pragma unroll
      for (int k = 0; k < kUnits; ++k) {
        const int m = (tid >> 3) + (GT / 8) * k;
        uint16_t* dst = nullptr;
        if (is_q) {
          if (q_out && ep.row_ok[m]) dst = q_out + ((size_t)(m0 + m) * hq + head) * 128;
        } else {
          const int page = ep.row_page[m];
          if (page >= 0) dst = kpool + (((size_t)page * hkv + g) * kPage + ep.row_slot[m]) * 128;
        }
        float olo[8], ohi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float lo = ep.c[m][c * 8 + e], hi = ep.c[m][64 + c * 8 + e];
          const float cs = tabv[k][e >> 1][2 * (e & 1)], sn = tabv[k][e >> 1][2 * (e & 1) + 1];
          olo[e] = lo * cs - hi * sn;
          ohi[e] = lo * sn + hi * cs;
        }
        u32x4 plo, phi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          plo[e] = pack_bf2(olo[2 * e], olo[2 * e + 1]);
          phi[e] = pack_bf2(ohi[2 * e], ohi[2 * e + 1]);
        }
        if (dst) {
          *reinterpret_cast<u32x4*>(dst + c * 8) = plo;
          *reinterpret_cast<u32x4*>(dst + 64 + c * 8) = phi;
        }
      }
    } else {
      // V head: page layout [d][slot]; thread tid takes output row tid % 256
      // and half of its 128 d (2-byte stores 32 bytes apart in its page).
      const int g = head - hq - hkv;
      constexpr int kDim = 128 * BM2 / GT;     // head dimensions per thread
      const int row = tid % BM2, e0 = (tid / BM2) * kDim;
      const int page = ep.row_page[row];
      if (page >= 0) {
        uint16_t* base = vpool + ((size_t)page * hkv + g) * 128 * kPage + ep.row_slot[row];
#pragma unroll 4
        for (int e = e0; e < e0 + kDim; e += 4) {
          const f32x4 c4 = *reinterpret_cast<const f32x4*>(&ep.c[row][e]);
#pragma unroll
          for (int i = 0; i < 4; ++i) base[(e + i) * kPage] = f2bf(c4[i]);
        }
      }
    }
  };
  auto epilogue = [&](auto wn_tag) __attribute__((always_inline)) {
    constexpr int WN = decltype(wn_tag)::value;
#pragma unroll
    for (int hi = 0; hi < HPT; ++hi) {
      const int h = HPT == 3 ? (hi == 0 ? 1 : hi == 1 ? 0 : 2) : hi;
      if (hi > 0) __syncthreads();             // every thread done with the previous head
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = WN * Cfg::WCOLS + j * 32;   // first tile column of this 32-column block
        if (col / BN != h) continue;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = wm * WROWS + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            ep.c[r][col % BN + (lane & 31)] = acc[i][j][v];
          }
      }
      __syncthreads();
      store_head(head1 + h);
    }
  };
  static_assert(Cfg::WGN == 2 || Cfg::WGN == 4, "wave columns");
  if (wn == 0) {
    epilogue(std::integral_constant<int, 0>{});
  } else if (wn == 1) {
    epilogue(std::integral_constant<int, 1>{});
  } else if constexpr (Cfg::WGN == 4) {
    if (wn == 2) epilogue(std::integral_constant<int, 2>{});
    else epilogue(std::integral_constant<int, 3>{});
  }
}

// bf16 path for a few rows (at most 64: a decode step's new tokens, a small
// Sparse-Q set): reading W dominates, so the work is spread over columns
// and the reduction dimension instead of row tiles.  Workgroup (head,
// quarter q) owns the 16 rotate-half pairs (16q + j, 64 + 16q + j) of one
// head, i.e. 32 output columns: RoPE pairs stay inside the workgroup.  Its
// 8 waves take interleaved 32-wide k-steps (v_mfma_f32_16x16x32_bf16: A =
// x rows, B = the 32 W rows), each with the operands of 8 k-steps in flight,
// and are summed in LDS in wave order.  RB row blocks of 16 share each W
// fragment.
constexpr int kSkWaves = 8, kSkThreads = 64 * kSkWaves;
template <int RB>
__global__ __launch_bounds__(kSkThreads) void qkv_skinny_bf16(
    const uint16_t* __restrict__ x, int hidden, const int32_t* __restrict__ rows, int n_rows,
    const uint16_t* __restrict__ w, int head0, sx_layout lay, int n_pages,
    uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool, uint16_t* __restrict__ q_out,
    int hq, int hkv) {
  constexpr int NR = 16 * RB;
  __shared__ float red[kSkWaves][NR][33];
  __shared__ int32_t s_tok[NR], s_ok[NR], s_page[NR], s_slot[NR], s_pos[NR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = head0 + blockIdx.x / 4, qd = blockIdx.x % 4;
  if (tid < NR) {
    int tok = tid < n_rows ? rows[tid] : -1;
    const int r = tok >= 0 ? find_request(lay.seq_start, lay.n_req, tok) : -1;
    const int idx = r >= 0 ? tok - lay.seq_start[r] : 0;
    s_ok[tid] = r >= 0;
    s_tok[tid] = (tok >= 0 && tok < lay.n_tok) ? tok : 0;   // rows past n_rows read token 0
    s_page[tid] = r >= 0 ? page_of(lay, n_pages, r, idx) : -1;
    s_slot[tid] = idx & (kPage - 1);
    s_pos[tid] = r >= 0 ? rope_pos(lay, r, idx) : 0;
  }
  __syncthreads();
  const int lr = lane & 15, lq = lane >> 4;
  // this lane's A rows (one per row block) and B rows (one per column block)
  const uint16_t* xa[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) xa[rb] = x + (size_t)s_tok[16 * rb + lr] * hidden + 8 * lq;
  const uint16_t* wb[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
    wb[cb] = w + ((size_t)head * 128 + 64 * cb + 16 * qd + lr) * hidden + 8 * lq;
  f32x4 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n_ks = hidden / 32;
  constexpr int U = 8;                       // k-steps whose operands are loaded together
  int ks = wave;
  for (; ks + kSkWaves * (U - 1) < n_ks; ks += kSkWaves * U) {
    bf16x8 a[U][RB], b[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (ks + kSkWaves * u) * 32;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) a[u][rb] = *reinterpret_cast<const bf16x8*>(xa[rb] + k);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) b[u][cb] = *reinterpret_cast<const bf16x8*>(wb[cb] + k);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][rb], b[u][cb], acc[rb][cb], 0, 0, 0);
  }
  for (; ks < n_ks; ks += kSkWaves) {
    const int k = ks * 32;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *reinterpret_cast<const bf16x8*>(xa[rb] + k), *reinterpret_cast<const bf16x8*>(wb[cb] + k),
            acc[rb][cb], 0, 0, 0);
  }
  // D: row 4*lq + v of the row block, column lr of the column block
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][16 * rb + 4 * lq + v][16 * cb + lr] = acc[rb][cb][v];
  __syncthreads();
  // one rotate-half pair (row m, e = 16 qd + j) per thread and step
  for (int u = tid; u < NR * 16; u += kSkThreads) {
    const int m = u >> 4, j = u & 15;
    if (m >= n_rows || !s_ok[m]) continue;
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int ww = 0; ww < kSkWaves; ++ww) {
      lo += red[ww][m][j];
      hi += red[ww][m][16 + j];
    }
    const int e = 16 * qd + j;
    if (head < hq + hkv) {
      const float* tab = lay.rope_tab + (size_t)s_pos[m] * 128 + 2 * e;
      const float cs = tab[0], sn = tab[1];
      const float olo = lo * cs - hi * sn, ohi = lo * sn + hi * cs;
      uint16_t* dst = nullptr;
      if (head < hq) {
        if (q_out) dst = q_out + ((size_t)m * hq + head) * 128;
      } else if (s_page[m] >= 0) {
        dst = kpool + (((size_t)s_page[m] * hkv + (head - hq)) * kPage + s_slot[m]) * 128;
      }
      if (dst) {
        dst[e] = f2bf(olo);
        dst[64 + e] = f2bf(ohi);
      }
    } else if (s_page[m] >= 0) {
      uint16_t* dst = vpool + ((size_t)s_page[m] * hkv + (head - hq - hkv)) * 128 * kPage + s_slot[m];
      dst[e * kPage] = f2bf(lo);
      dst[(64 + e) * kPage] = f2bf(hi);
    }
  }
}

// fp32 storage: one workgroup per (row, head), one lane per rotate-half pair
// (or per element for V); dot products accumulate in index order.
template <int D>
__global__ __launch_bounds__(128) void qkv_rows_f32(
    const float* __restrict__ x, int hidden, const int32_t* __restrict__ rows, int n_rows,
    const float* __restrict__ w, int head0, sx_layout lay, int n_pages, float* __restrict__ kpool,
    float* __restrict__ vpool, float* __restrict__ q_out, int hq, int hkv) {
  extern __shared__ float xs[];
  const int m = blockIdx.x;
  const int head = head0 + blockIdx.y;
  const int tok = rows[m];
  const int r = find_request(lay.seq_start, lay.n_req, tok);
  if (r < 0) return;
  const int idx = tok - lay.seq_start[r];
  for (int c = threadIdx.x; c < hidden; c += blockDim.x) xs[c] = x[(size_t)tok * hidden + c];
  __syncthreads();
  const float* wt = w + (size_t)head * D * hidden;
  if (head < hq + hkv) {
    const int e = threadIdx.x;
    if (e >= D / 2) return;
    float lo = 0.f, hi = 0.f;
    for (int c = 0; c < hidden; ++c) {
      lo = fmaf(xs[c], wt[(size_t)e * hidden + c], lo);
      hi = fmaf(xs[c], wt[(size_t)(e + D / 2) * hidden + c], hi);
    }
    const float* tab = lay.rope_tab + (size_t)rope_pos(lay, r, idx) * D + 2 * e;
    const float olo = lo * tab[0] - hi * tab[1];
    const float ohi = lo * tab[1] + hi * tab[0];
    float* dst;
    if (head < hq) {
      if (!q_out) return;
      dst = q_out + ((size_t)m * hq + head) * D;
    } else {
      const int page = page_of(lay, n_pages, r, idx);
      if (page < 0) return;
      dst = kpool + (((size_t)page * hkv + (head - hq)) * kPage + (idx & (kPage - 1))) * D;
    }
    dst[e] = olo;
    dst[e + D / 2] = ohi;
  } else {
    const int page = page_of(lay, n_pages, r, idx);
    if (page < 0) return;
    const int g = head - hq - hkv;
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
      float s = 0.f;
      for (int c = 0; c < hidden; ++c) s = fmaf(xs[c], wt[(size_t)e * hidden + c], s);
      vpool[(((size_t)page * hkv + g) * D + e) * kPage + (idx & (kPage - 1))] = s;
    }
  }
}

// Heads per tile: one workgroup fills a compute unit (256 of them), so a
// launch takes about ceil(tiles / 256) rounds, and a round of two-head tiles
// costs about 1.7 rounds of one-head tiles, one of three-head tiles about
// 2.6 (measured at 870 to 31,488 rows: the per-tile time grows less than
// the work because fewer bytes are staged per flop).  The launcher takes the
// cheapest, e.g. three heads for 3,379 rows (224 tiles, one round: 0.228
// against 0.240 ms with one head), two for 13,824 or 31,488 rows, one for a
// few hundred.
constexpr int kGemmCUs = 256;
int gemm_heads_per_tile(int mt, int n_heads) {
  static const int cost10[4] = {0, 10, 17, 26};
  int best = 1;
  long long best_cost = -1;
  for (int hpt = 1; hpt <= 3; ++hpt) {
    if (n_heads % hpt != 0) continue;
    const long long tiles = (long long)mt * (n_heads / hpt);
    const long long cost = (tiles + kGemmCUs - 1) / kGemmCUs * cost10[hpt];
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = hpt;
    }
  }
  return best;
}

}  // namespace

namespace {

// The projection of rows, with (side != nullptr) the realign jobs of another
// pool in the same launch when the tiles leave at least kMinRealignWorkers
// compute units free; *fused tells the caller whether they were.
constexpr int kMinRealignWorkers = 16;
sx_status launch_recompute_impl(const sx_dims& dims, const sx_layout& lay, const void* x,
                                const int32_t* rows, int n_rows, const void* w_qkv,
                                const sx_pages& kv, void* q_out, SideRealign* side, bool* fused,
                                hipStream_t stream) {
  *fused = false;
  if (n_rows == 0) return SX_OK;
  const int hq = dims.n_q_heads, hkv = dims.n_kv_heads;
  const int head0 = q_out ? 0 : hq;
  const int n_heads = hq + 2 * hkv - head0;
  if (dims.dtype == SX_BF16 && n_rows <= 64) {
    const dim3 grid(n_heads * 4);
    auto go = [&](auto kernel) {
      kernel<<<grid, kSkThreads, 0, stream>>>(
          (const uint16_t*)x, dims.hidden, rows, n_rows, (const uint16_t*)w_qkv, head0, lay, kv.n_pages,
          (uint16_t*)kv.k, (uint16_t*)kv.v, (uint16_t*)q_out, hq, hkv);
    };
    if (n_rows <= 16) go(qkv_skinny_bf16<1>);
    else if (n_rows <= 32) go(qkv_skinny_bf16<2>);
    else if (n_rows <= 48) go(qkv_skinny_bf16<3>);
    else go(qkv_skinny_bf16<4>);
  } else if (dims.dtype == SX_BF16) {
    const int mt = (n_rows + BM2 - 1) / BM2;
    auto go = [&](auto kernel, int hpt, size_t smem) -> sx_status {
      const int nt = n_heads / hpt;
      const int grid = ((mt * nt + 7) / 8) * 8;
      SideRealign none = {};
      none.tile_blocks = grid;
      int workers = 0;
      if (side && side->n_jobs > 0 && kGemmCUs - grid >= kMinRealignWorkers) {
        workers = kGemmCUs - grid;
        side->tile_blocks = grid;
        *fused = true;
      }
      const sx_status st = allow_lds((const void*)kernel, smem, "sx_recompute_kv");
      if (st != SX_OK) return st;
      kernel<<<grid + workers, GT, smem, stream>>>(
          (const uint16_t*)x, dims.hidden, rows, n_rows, (const uint16_t*)w_qkv, head0, mt, nt,
          lay, kv.n_pages, (uint16_t*)kv.k, (uint16_t*)kv.v, (uint16_t*)q_out, hq, hkv,
          workers ? *side : none);
      return SX_OK;
    };
    const int hpt = gemm_heads_per_tile(mt, n_heads);
    const sx_status st = hpt == 3   ? go(qkv_gemm256_bf16<3>, 3, sizeof(Gemm2Smem<3>))
                         : hpt == 2 ? go(qkv_gemm256_bf16<2>, 2, sizeof(Gemm2Smem<2>))
                                    : go(qkv_gemm256_bf16<1>, 1, sizeof(Gemm2Smem<1>));
    if (st != SX_OK) return st;
  } else {
    dim3 grid(n_rows, n_heads);
    const size_t smem = (size_t)dims.hidden * sizeof(float);
    if (dims.head_dim == 64)
      qkv_rows_f32<64><<<grid, 128, smem, stream>>>((const float*)x, dims.hidden, rows, n_rows,
                                                    (const float*)w_qkv, head0, lay, kv.n_pages,
                                                    (float*)kv.k, (float*)kv.v, (float*)q_out, hq, hkv);
    else
      qkv_rows_f32<128><<<grid, 128, smem, stream>>>((const float*)x, dims.hidden, rows, n_rows,
                                                     (const float*)w_qkv, head0, lay, kv.n_pages,
                                                     (float*)kv.k, (float*)kv.v, (float*)q_out, hq, hkv);
  }
  return check_launch("sx_recompute_kv");
}

}  // namespace

sx_status launch_recompute(const sx_dims& dims, const sx_layout& lay, const void* x,
                           const int32_t* rows, int n_rows, const void* w_qkv,
                           const sx_pages& kv, void* q_out, hipStream_t stream) {
  bool fused;
  return launch_recompute_impl(dims, lay, x, rows, n_rows, w_qkv, kv, q_out, nullptr, &fused, stream);
}

// sx_recompute_kv of kv plus sx_rope_realign of rsrc -> rdst, which the
// caller guarantees writes pages the projection does not touch.  One launch
// when the projection's tiles leave compute units free (bf16, more than 64
// rows, fewer than kGemmCUs - kMinRealignWorkers tiles): the realign jobs
// run on those.  Otherwise the two launch one after the other.
sx_status launch_recompute_realign(const sx_dims& dims, const sx_layout& lay, const void* x,
                                   const int32_t* rows, int n_rows, const void* w_qkv,
                                   const sx_pages& kv, void* q_out, const sx_pages& rsrc,
                                   const sx_pages& rdst, const sx_realign_job* jobs, int n_jobs,
                                   hipStream_t stream) {
  SideRealign side = {};
  if (dims.dtype == SX_BF16 && dims.head_dim == 128) {
    side.ksrc = (const uint16_t*)rsrc.k;
    side.vsrc = (const uint16_t*)rsrc.v;
    side.kdst = (uint16_t*)rdst.k;
    side.vdst = (uint16_t*)rdst.v;
    side.jobs = jobs;
    side.n_src_pages = rsrc.n_pages;
    side.n_dst_pages = rdst.n_pages;
    side.n_jobs = n_jobs;
  }
  bool fused = false;
  const sx_status st = launch_recompute_impl(dims, lay, x, rows, n_rows, w_qkv, kv, q_out,
                                             side.n_jobs > 0 ? &side : nullptr, &fused, stream);
  if (st != SX_OK || fused) return st;
  return launch_realign(dims, lay, rsrc, rdst, jobs, n_jobs, stream);
}

}  // namespace sx
