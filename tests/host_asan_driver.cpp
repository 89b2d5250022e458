// Host-side driver for the AddressSanitizer / UBSan build of libsx's host
// code (api.cpp: argument checks and the planners; seg_index.cpp: the
// segment index).  Built with g++ and run on the CPU by tests/test_host_asan.py.
// Every buffer is allocated at exactly the size sx.h documents, so a write
// past it is reported.  The device launchers are replaced by stubs that abort:
// every device call made here must be rejected by the argument checks before
// anything would be launched.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "sx.h"
#include "sx_internal.hpp"

// ---- stubs for the device side (never reached) -----------------------------
namespace sx {
[[noreturn]] static void reached(const char* what) {
  std::fprintf(stderr, "device launcher reached from a call that should have failed: %s\n", what);
  std::abort();
}
size_t attn_ws_bytes(const sx_dims&, int, int, bool) { return size_t(1) << 20; }
size_t topk_ws_bytes(int, int) { return size_t(1) << 20; }
size_t select_ws_bytes(const sx_dims&, int, int, int) { return size_t(1) << 20; }
size_t decode_ws_bytes(const sx_dims&, int, int) { return size_t(1) << 20; }
size_t decode_noalloc_capacity() { return size_t(4) << 20; }
int score_parts(const sx_dims& d, int, int) { return d.n_kv_heads; }
sx_status decode_scratch(void**) { reached("decode_scratch"); }
bool debug_enabled() { return false; }
DebugCheck::DebugCheck(hipStream_t, const char*) { reached("DebugCheck"); }
void DebugCheck::layout(const sx_layout&, int, bool) { reached("DebugCheck::layout"); }
void DebugCheck::rows(const int32_t*, const int32_t*, int, const sx_layout&) { reached("DebugCheck::rows"); }
void DebugCheck::jobs(const sx_realign_job*, int, int, int, int) { reached("DebugCheck::jobs"); }
sx_status DebugCheck::finish() { reached("DebugCheck::finish"); }
sx_status launch_realign(const sx_dims&, const sx_layout&, const sx_pages&, const sx_pages&,
                         const sx_realign_job*, int, hipStream_t) { reached("launch_realign"); }
sx_status launch_recompute(const sx_dims&, const sx_layout&, const void*, const int32_t*, int,
                           const void*, const sx_pages&, void*, hipStream_t) { reached("launch_recompute"); }
sx_status launch_recompute_realign(const sx_dims&, const sx_layout&, const void*, const int32_t*, int,
                                   const void*, const sx_pages&, void*, const sx_pages&, const sx_pages&,
                                   const sx_realign_job*, int, hipStream_t) {
  reached("launch_recompute_realign");
}
sx_status launch_attention(const sx_dims&, const sx_layout&, const void*, const int32_t*, const int32_t*,
                           const int32_t*, int, const sx_pages&, void*, float*, void*, hipStream_t) {
  reached("launch_attention");
}
sx_status launch_attention_plan(const sx_dims&, const sx_layout&, const int32_t*, const int32_t*, int,
                                void*, hipStream_t) { reached("launch_attention_plan"); }
sx_status launch_attention_run(const sx_dims&, const sx_layout&, const void*, const int32_t*,
                               const int32_t*, int, const sx_pages&, void*, float*, void*, hipStream_t) {
  reached("launch_attention_run");
}
sx_status launch_decode(const sx_dims&, const sx_layout&, const void*, const sx_pages&, void*, float*,
                        void*, hipStream_t) { reached("launch_decode"); }
sx_status launch_scores(const sx_dims&, const sx_layout&, const void*, const int32_t*, const int32_t*,
                        const int32_t*, int, const float*, const int32_t*, const sx_pages&, float*,
                        void*, hipStream_t) { reached("launch_scores"); }
size_t scores_gather_bytes(const sx_dims&, int) { return 0; }
sx_status launch_topk(const float*, int, const uint8_t*, const int32_t*, int, int, const int32_t*,
                      const int32_t*, int32_t*, int32_t*, float*, void*, hipStream_t) { reached("launch_topk"); }
sx_status launch_mfma_peak(int, int, int, float*, hipStream_t) { reached("launch_mfma_peak"); }
}  // namespace sx

// ---- checks ---------------------------------------------------------------
static int g_fail = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "%s:%d: check failed: %s (%s)\n", __FILE__, __LINE__, \
                   #cond, sx_last_error());                                      \
      ++g_fail;                                                                  \
    }                                                                            \
  } while (0)

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(uint32_t n) {   // xorshift64*, uniform enough for sizes
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return n ? (uint32_t)((g_rng * 2685821657736338717ull) >> 33) % n : 0;
}

static void rope_tables() {
  std::vector<float> tab(64 * 128);
  CHECK(sx_rope_table(1e4, 128, 64, tab.data()) == SX_OK);
  CHECK(sx_rope_table(-1.0, 128, 64, tab.data()) == SX_EINVAL);
  CHECK(sx_rope_table(1e4, 127, 64, tab.data()) == SX_EINVAL);
  CHECK(sx_rope_table(1e4, 128, 0, tab.data()) == SX_EINVAL);
  CHECK(sx_rope_table(1e4, 128, 64, nullptr) == SX_EINVAL);
}

static void plan_layouts() {
  for (int it = 0; it < 400; ++it) {
    const int n_req = 1 + (int)rnd(6);
    std::vector<int32_t> pstart(n_req + 1, 0), preuse, plen, num(n_req), den(n_req);
    for (int r = 0; r < n_req; ++r) {
      const int np = (int)rnd(9);
      for (int p = 0; p < np; ++p) {
        preuse.push_back((int32_t)rnd(2));
        plen.push_back((int32_t)rnd(300));
      }
      pstart[r + 1] = (int32_t)preuse.size();
      den[r] = 1 + (int32_t)rnd(1000);
      num[r] = (int32_t)rnd((uint32_t)den[r] + 1);
    }
    if (preuse.empty()) {   // keep the piece arrays non-empty for data()
      preuse.push_back(0);
      plen.push_back(0);
    }
    int64_t total = 0;
    for (int p = 0; p < pstart[n_req]; ++p) total += plen[p];
    const int cap = (int)total;
    std::vector<int32_t> seq(n_req + 1), sq(cap > 0 ? cap : 1), sqs(n_req + 1), ncand(n_req), k(n_req);
    std::vector<uint8_t> cls(cap > 0 ? cap : 1);
    const int fb = (int)rnd(80), ov = (int)rnd(3) * 8;
    CHECK(sx_plan_layout(n_req, pstart.data(), preuse.data(), plen.data(), num.data(), den.data(), fb,
                         ov, cap, seq.data(), cls.data(), sq.data(), sqs.data(), ncand.data(),
                         k.data()) == SX_OK);
    CHECK(seq[n_req] == cap);
    for (int r = 0; r < n_req; ++r) {
      int nc = 0;
      for (int j = seq[r]; j < seq[r + 1]; ++j) nc += cls[j] == 0;
      CHECK(nc == ncand[r]);
      CHECK(k[r] == (int32_t)(((int64_t)num[r] * nc) / den[r]));
      for (int i = sqs[r]; i < sqs[r + 1]; ++i) {
        CHECK(sq[i] >= seq[r] && sq[i] < seq[r + 1] && cls[sq[i]] == 1);
        if (i > sqs[r]) CHECK(sq[i] > sq[i - 1]);
      }
    }
    // one token short of the batch: rejected, nothing written past the buffers
    if (cap > 0) {
      std::vector<int32_t> sq2(cap - 1 > 0 ? cap - 1 : 1);
      std::vector<uint8_t> cls2(cap - 1 > 0 ? cap - 1 : 1);
      CHECK(sx_plan_layout(n_req, pstart.data(), preuse.data(), plen.data(), num.data(), den.data(),
                           fb, ov, cap - 1, seq.data(), cls2.data(), sq2.data(), sqs.data(),
                           ncand.data(), k.data()) == SX_EINVAL);
    }
  }
}

static void plan_realigns() {
  for (int it = 0; it < 300; ++it) {
    const int n_req = 1 + (int)rnd(3), max_pages = 8 + (int)rnd(40);
    std::vector<int32_t> bt((size_t)n_req * max_pages);
    for (auto& v : bt) v = (int32_t)rnd(5000);
    const int n_segs = (int)rnd(6);
    std::vector<sx_segment> segs(n_segs > 0 ? n_segs : 1);
    int n_ids = 0;
    for (int s = 0; s < n_segs; ++s) {
      sx_segment& g = segs[s];
      g.req = (int32_t)rnd(n_req);
      g.len = (int32_t)rnd(120);
      g.dst_start = (int32_t)rnd((uint32_t)(max_pages * 16 - g.len));
      g.p_src = (int32_t)rnd(4000);
      g.src_slot0 = (int32_t)rnd(16);
      g.src_pages_off = n_ids;
      n_ids += (g.src_slot0 + g.len + 15) / 16 + 1;
    }
    std::vector<int32_t> ids(n_ids > 0 ? n_ids : 1);
    for (auto& v : ids) v = (int32_t)rnd(5000);
    const int bound = sx_realign_jobs_bound(segs.data(), n_segs, 16);
    std::vector<sx_realign_job> jobs(bound > 0 ? bound : 1);
    int n_jobs = -1;
    CHECK(sx_plan_realign(segs.data(), n_segs, ids.data(), n_ids, bt.data(), n_req, max_pages, 16, nullptr,
                          jobs.data(), bound, &n_jobs) == SX_OK);
    int covered = 0, want = 0;
    for (int s = 0; s < n_segs; ++s) want += segs[s].len;
    for (int j = 0; j < n_jobs; ++j) {
      CHECK(jobs[j].n_tok > 0 && jobs[j].src_slot + jobs[j].n_tok <= 16 && jobs[j].dst_slot + jobs[j].n_tok <= 16);
      covered += jobs[j].n_tok;
    }
    CHECK(n_jobs >= 0 && covered == want);
    if (n_jobs > 1) {
      std::vector<sx_realign_job> small(n_jobs - 1);
      CHECK(sx_plan_realign(segs.data(), n_segs, ids.data(), n_ids, bt.data(), n_req, max_pages, 16,
                            nullptr, small.data(), n_jobs - 1, &n_jobs) == SX_EINVAL);
    }
  }
}

static void segment_index() {
  for (int round = 0; round < 6; ++round) {
    const int n_blocks = 64 + (int)rnd(200), bs = 16;
    sx_index* ix = nullptr;
    CHECK(sx_index_create(n_blocks, bs, 9, 10, &ix) == SX_OK && ix);
    if (!ix) return;
    std::vector<std::vector<int32_t>> held;   // blocks we hold a reference on
    for (int step = 0; step < 3000; ++step) {
      const int op = (int)rnd(6);
      if (op == 0) {                           // allocate and register a segment
        const int n_tok = 1 + (int)rnd(5 * bs);
        const int nb = (n_tok + bs - 1) / bs;
        std::vector<int32_t> ids(nb), toks(n_tok);
        for (auto& t : toks) t = (int32_t)rnd(50);
        const sx_status st = sx_index_alloc(ix, nb, ids.data());
        CHECK(st == SX_OK || st == SX_ENOMEM);
        if (st == SX_OK) {
          CHECK(sx_index_insert(ix, toks.data(), n_tok, rnd(3), ids.data(), (int32_t)rnd(1000),
                                (int32_t)rnd(2)) == SX_OK);
          held.push_back(ids);
        }
      } else if (op == 1 && !held.empty()) {   // release one held list
        const size_t i = rnd((uint32_t)held.size());
        CHECK(sx_index_release(ix, held[i].data(), (int32_t)held[i].size()) == SX_OK);
        held.erase(held.begin() + (long)i);
      } else if (op == 2) {                    // look up a random segment, then plan it
        const int n_tok = (int)rnd(6 * bs);
        const int nb = n_tok / bs;
        std::vector<int32_t> toks(n_tok > 0 ? n_tok : 1), blk(nb > 0 ? nb : 1), pos(nb > 0 ? nb : 1);
        for (auto& t : toks) t = (int32_t)rnd(50);
        CHECK(sx_index_lookup(ix, toks.data(), n_tok, rnd(3), blk.data(), pos.data()) == SX_OK);
        std::vector<int32_t> hits;
        for (int j = 0; j < nb; ++j)
          if (blk[j] >= 0) hits.push_back(blk[j]);
        std::vector<sx_segment> segs(nb + 1);
        std::vector<int32_t> sids(nb + 1), pre(nb + 1), plen(nb + 1);
        int32_t n_segs = 0, n_ids = 0, n_pieces = 0;
        CHECK(sx_plan_segments(0, 0, blk.data(), pos.data(), n_tok, bs, 0, segs.data(), &n_segs,
                               sids.data(), &n_ids, pre.data(), plen.data(), &n_pieces) == SX_OK);
        CHECK(n_ids == (int32_t)hits.size());
        if (!hits.empty()) CHECK(sx_index_release(ix, hits.data(), (int32_t)hits.size()) == SX_OK);
      } else if (op == 3 && !held.empty()) {   // delete a segment's blocks from the index
        const size_t i = rnd((uint32_t)held.size());
        CHECK(sx_index_remove(ix, held[i].data(), (int32_t)held[i].size()) == SX_OK);
      } else if (op == 4) {
        int32_t stats[4];
        CHECK(sx_index_stats(ix, stats) == SX_OK);
        CHECK(stats[0] + stats[1] == n_blocks);
      } else {                                 // bad ids are rejected
        int32_t bad[2] = {-1, n_blocks + 3};
        CHECK(sx_index_release(ix, bad, 2) == SX_EINVAL);
      }
    }
    sx_index_destroy(ix);
  }
  uint64_t h = 0;
  std::vector<int32_t> toks(100);
  for (int n = 0; n <= 100; ++n) CHECK(sx_virtual_hash(toks.data(), n, 7, &h) == SX_OK);
}

static void device_entry_validation() {
  sx_dims d = {4096, 32, 8, 128, 16, SX_BF16};
  int32_t fake_i[4] = {0, 16, 0, 0};
  float fake_f[4] = {0, 0, 0, 0};
  sx_layout lay = {1, 16, 1, 16, fake_i, fake_i, nullptr, fake_f};
  sx_pages pages = {fake_f, fake_f, 4};
  char ws[8];
  CHECK(sx_recompute_kv(nullptr, &lay, fake_f, fake_i, 1, fake_f, &pages, nullptr, nullptr) == SX_EINVAL);
  sx_dims bad = d;
  bad.head_dim = 64;
  CHECK(sx_sparse_attn(&bad, &lay, fake_f, fake_i, fake_i, 1, &pages, fake_f, nullptr, ws, sizeof ws,
                       nullptr) == SX_EUNSUPPORTED);
  CHECK(sx_sparse_attn(&d, &lay, fake_f, fake_i, fake_i, 100, &pages, fake_f, nullptr, ws, sizeof ws,
                       nullptr) == SX_EWORKSPACE);
  CHECK(sx_full_attn(&d, &lay, fake_f, &pages, fake_f, nullptr, ws, sizeof ws, nullptr) == SX_EWORKSPACE);
  CHECK(sx_decode_attn(&d, &lay, fake_f, &pages, fake_f, nullptr, ws, sizeof ws, nullptr) == SX_EWORKSPACE);
  sx_layout empty_bt = lay;
  empty_bt.max_pages = 0;
  CHECK(sx_decode_attn_noalloc(&d, &empty_bt, fake_f, &pages, fake_f, nullptr, nullptr) == SX_EINVAL);
  CHECK(sx_rope_realign(&d, &lay, &pages, &pages, nullptr, 3, nullptr) == SX_EINVAL);
  sx_pages other = {fake_i, fake_i, 4};
  CHECK(sx_recompute_kv_realign(&d, &lay, fake_f, fake_i, 1, fake_f, &pages, nullptr, &other, &pages,
                                nullptr, 1, nullptr) == SX_EINVAL);
  CHECK(sx_recompute_kv_realign(&d, &lay, fake_f, fake_i, 1, fake_f, &pages, nullptr, &pages, &other,
                                nullptr, 1, nullptr) == SX_EINVAL);
  CHECK(sx_select_topk(&d, &lay, fake_f, nullptr, fake_i, fake_i, 4, nullptr, &pages, nullptr, fake_i,
                       fake_i, nullptr, nullptr, ws, sizeof ws, nullptr) == SX_EINVAL);
  CHECK(sx_topk(nullptr, nullptr, fake_i, 1, 4, fake_i, fake_i, nullptr, 0, nullptr) == SX_EINVAL);
  CHECK(sx_mfma_peak_probe(0, 1, 0, fake_f, nullptr) == SX_EINVAL);
  CHECK(std::strlen(sx_last_error()) > 0);
}

int main() {
  rope_tables();
  plan_layouts();
  plan_realigns();
  segment_index();
  device_entry_validation();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host driver: all checks passed\n");
  return 0;
}
