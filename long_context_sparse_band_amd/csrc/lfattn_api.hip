// C-ABI entry points of liblfattn (declared in include/lfattn.h): argument
// checks, the canonical global list, the band work table, workspace, and the
// kernel launches.
#include "lfattn.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "lfattn_internal.h"

using lfattn::BandWork;
using lfattn::kBandRows;
using lfattn::kTileKeys;
using lfattn::kWaveRows;

namespace {

constexpr int kMaxTimedForwards = 4096;
// Timing events per forward: band start/stop, global partials start/stop,
// merge start/stop.
constexpr int kEvPerForward = 6;
constexpr int kXcds = 8;           // MI355X: workgroups go round-robin over 8 XCDs
constexpr int kMaxChunks = lfattn::kMergeBatch;  // key chunks per global row set
constexpr int kGlobTarget = 1024;  // aim for this many global-row workgroups
// Keys per global-row item of the band launch: short items when the whole
// launch fits one round of workgroup slots (they then set the critical
// path), longer ones otherwise (fewer items, less per-item overhead).
constexpr int kGlobItemKeysShort = 256, kGlobItemKeysLong = 512;
constexpr int kWideRounds = 2;
constexpr long long kMaxN = 1LL << 29;

}  // namespace

struct lfattn_ctx {
  int B = 0, H = 0, N = 0, D = 0, dtype = 0, window = 0, hw = 0;
  float scale = 0.0f;
  std::vector<int> dil;
  std::vector<int> glob;  // sorted, unique
  long long pairs = 0;
  int device = 0;

  BandWork* d_work = nullptr;
  int n_band_wg = 0;
  int* d_glob = nullptr;
  unsigned char* d_isglob = nullptr;

  float* d_part = nullptr;
  int band_rows = 0;  // rows per band workgroup
  int g_waves = 0, g_rows = 0, n_sets = 0, n_chunks = 0, chunk_keys = 0, n_glob_wg = 0;
  bool glob_items = false;  // global-row partials run as items of the band launch

  bool timing = false;
  int n_timed = 0;
  std::vector<hipEvent_t> ev;  // kEvPerForward per timed forward
};

namespace {

template <typename T>
lfattn_status dev_alloc(T** p, size_t count) {
  *p = nullptr;
  if (count == 0) return LFATTN_OK;
  if (hipMalloc((void**)p, count * sizeof(T)) != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return LFATTN_ENOMEM;
  }
  return LFATTN_OK;
}

void free_ctx(lfattn_ctx* c) {
  if (!c) return;
  (void)hipFree(c->d_work);
  (void)hipFree(c->d_glob);
  (void)hipFree(c->d_isglob);
  (void)hipFree(c->d_part);
  for (hipEvent_t e : c->ev) (void)hipEventDestroy(e);
  delete c;
}

// Scored pairs of one head with dilation d: every row's band (keys i + d*k,
// |k| <= hw, inside [0, N)), plus the global keys outside that band; global
// rows score all N keys.
long long head_pairs(int N, long long hw, int d, const std::vector<int>& glob,
                     const std::vector<unsigned char>& isg) {
  long long total = 0;
  for (long long i = 0; i < N; ++i) {
    if (isg[i]) {
      total += N;
      continue;
    }
    long long left = std::min(i / d, hw), right = std::min((N - 1 - i) / d, hw);
    long long n = 1 + left + right;
    for (int g : glob) {
      long long off = g - i;
      bool in_band = off % d == 0 && off / d <= hw && off / d >= -hw;
      if (!in_band) ++n;
    }
    total += n;
  }
  return total;
}

bool overlaps(const void* a, const void* b, size_t bytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bytes && y < x + bytes;
}

}  // namespace

extern "C" {

const char* lfattn_status_string(lfattn_status s) {
  switch (s) {
    case LFATTN_OK: return "ok";
    case LFATTN_EINVAL: return "invalid argument";
    case LFATTN_EUNSUPPORTED: return "unsupported configuration";
    case LFATTN_ENOMEM: return "out of memory";
    case LFATTN_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

lfattn_status lfattn_create(lfattn_t* out, int B, int H, int N, int D, lfattn_dtype dtype,
                            int window, const int* dilation, const int* global_idx,
                            int n_global, float scale) {
  // ---- argument checks: no HIP call before all of them pass ----
  if (!out) return LFATTN_EINVAL;
  *out = nullptr;
  if (B < 1 || H < 1 || N < 1 || D < 1 || window < 0 || n_global < 0) return LFATTN_EINVAL;
  if (dtype != LFATTN_F32 && dtype != LFATTN_BF16) return LFATTN_EINVAL;
  if (n_global > 0 && !global_idx) return LFATTN_EINVAL;
  if (std::isnan(scale) || std::isinf(scale)) return LFATTN_EINVAL;
  if (dilation)
    for (int h = 0; h < H; ++h)
      if (dilation[h] < 1) return LFATTN_EINVAL;
  for (int t = 0; t < n_global; ++t)
    if (global_idx[t] < 0 || global_idx[t] >= N) return LFATTN_EINVAL;
  if (D != 64 && D != 128) return LFATTN_EUNSUPPORTED;
  if ((long long)N >= kMaxN || (long long)B * H > (1LL << 24)) return LFATTN_EUNSUPPORTED;

  lfattn_ctx* c = new (std::nothrow) lfattn_ctx;
  if (!c) return LFATTN_ENOMEM;
  c->B = B; c->H = H; c->N = N; c->D = D; c->dtype = (int)dtype; c->window = window;
  c->hw = (int)std::min<long long>(window / 2, N);  // a wider half-width changes nothing
  c->scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
  c->dil.assign(H, 1);
  if (dilation) c->dil.assign(dilation, dilation + H);
  // Canonical global list: sorted, repeats removed (a position listed twice is
  // global once, as setting a mask row or column twice changes nothing).
  c->glob.assign(global_idx, global_idx + n_global);
  std::sort(c->glob.begin(), c->glob.end());
  c->glob.erase(std::unique(c->glob.begin(), c->glob.end()), c->glob.end());
  if (dtype == LFATTN_BF16 && (int)c->glob.size() > lfattn::kMaxGlobalBf16) {
    delete c;
    return LFATTN_EUNSUPPORTED;
  }
  std::vector<unsigned char> isg(N, 0);
  for (int g : c->glob) isg[g] = 1;

  // Scored pairs, per distinct dilation value.
  {
    std::vector<int> ds = c->dil;
    std::sort(ds.begin(), ds.end());
    ds.erase(std::unique(ds.begin(), ds.end()), ds.end());
    long long total = 0;
    for (int d : ds) {
      long long per = head_pairs(N, window / 2, d, c->glob, isg);
      total += per * (long long)std::count(c->dil.begin(), c->dil.end(), d);
    }
    c->pairs = total * B;
  }

  // Compute units of the device (for sizing the work to one round of slots).
  int cus = 0;
  {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
      (void)hipGetLastError();
      cus = 256;
    }
  }
  const long long slots = (long long)lfattn::band_workgroups_per_cu(dtype, D) * cus;

  // Rows per band workgroup.  fp32: 128.  bf16: 64 (the workgroup's key tiles
  // split in two halves, each on its own pair of 32-row wavefronts: twice the
  // workgroups), or 128 (one tile stream shared by four 32-row blocks: half
  // the K/V loads per row) when there are enough 64-row blocks to fill the
  // slots kWideRounds times over.
  int band_rows = kBandRows;
  if (dtype == LFATTN_BF16) {
    long long n64 = 0;
    for (int h = 0; h < H; ++h) {
      const int d = c->dil[h];
      for (int r = 0; r < d && r < N; ++r) n64 += (long long)B * ((N - r + d - 1) / d + 63) / 64;
    }
    band_rows = n64 >= kWideRounds * slots ? 128 : 64;
    // LFATTN_BAND_ROWS=64 or 128 overrides the choice (both kernels give the
    // same results; this lets small problems exercise the 128-row one).
    if (const char* e = std::getenv("LFATTN_BAND_ROWS")) {
      if (std::strcmp(e, "64") == 0) band_rows = 64;
      if (std::strcmp(e, "128") == 0) band_rows = 128;
    }
  }
  c->band_rows = band_rows;

  // Band work: one item per workgroup's rows of each (b, h, residue r)
  // subsequence, laid out so that the items the hardware sends to one XCD
  // (blockIdx congruent mod 8) are consecutive query blocks of the same head,
  // which share their band's K and V rows in that XCD's L2.
  std::vector<BandWork> items;
  for (int bh = 0; bh < B * H; ++bh) {
    const int d = c->dil[bh % H];
    for (int r = 0; r < d && r < N; ++r) {
      const int Lr = (N - r + d - 1) / d;
      for (int t0 = 0; t0 < Lr; t0 += band_rows) items.push_back(BandWork{bh, r, t0, d});
    }
  }
  const int n_items = (int)items.size();
  std::vector<BandWork> table(n_items);
  // XCD that runs each band item, for placing the global-row items next to
  // the band items that read the same keys.
  std::vector<int> item_xcd(n_items);
  {
    int next = 0;
    for (int x = 0; x < kXcds; ++x)
      for (int bid = x; bid < n_items; bid += kXcds) {
        item_xcd[next] = x;
        table[bid] = items[next++];
      }
  }

  // Global rows: sets of rows (a workgroup's share of the global rows) times
  // key chunks.  bf16: each (b, h, row set, 256- or 512-key chunk) is one more
  // item at the end of the band launch, so that those workgroups are
  // dispatched last and fill the slots the band items leave free.  fp32: a
  // separate kernel (below).
  const int n_g = (int)c->glob.size();
  c->glob_items = n_g > 0 && lfattn::band_takes_global_items(dtype, D);
  if (c->glob_items) {
    c->g_rows = band_rows;  // a global item's rows: one workgroup's rows of G
    c->n_sets = (n_g + c->g_rows - 1) / c->g_rows;
    const long long short_items = (long long)B * H * c->n_sets *
                                  ((N + kGlobItemKeysShort - 1) / kGlobItemKeysShort);
    const int keys = n_items + short_items <= slots ? kGlobItemKeysShort : kGlobItemKeysLong;
    c->chunk_keys = keys;
    c->n_chunks = (N + keys - 1) / keys;
    // Each global item goes to the XCD of the residue-0 band item whose rows
    // start nearest its chunk (that XCD's L2 holds the chunk's K and V rows):
    // items are queued per XCD and dealt to block indices congruent to it,
    // falling back to another queue when one runs dry.
    std::vector<std::vector<BandWork>> q(kXcds);
    std::vector<int> first_item(B * H, -1);
    for (int k = 0; k < n_items; ++k)
      if (first_item[items[k].bh] < 0) first_item[items[k].bh] = k;
    for (int bh = 0; bh < B * H; ++bh)
      for (int set = 0; set < c->n_sets; ++set)
        for (int ch = 0; ch < c->n_chunks; ++ch) {
          const int d = c->dil[bh % H];
          const long long key0 = (long long)ch * keys;
          // residue 0's items come first for this head; its subsequence
          // position of key0 is key0 / d.
          const int k = std::min(first_item[bh] + (int)(key0 / d / band_rows), n_items - 1);
          q[item_xcd[std::max(k, 0)]].push_back(BandWork{bh, set, ch, 0});
        }
    size_t left = 0;
    for (auto& v : q) left += v.size();
    std::vector<size_t> pos(kXcds, 0);
    while (left > 0) {
      int x = (int)(table.size() % kXcds);
      for (int t = 0; t < kXcds && pos[x] >= q[x].size(); ++t) x = (x + 1) % kXcds;
      table.push_back(q[x][pos[x]++]);
      --left;
    }
  } else if (n_g > 0) {
    // fp32: a separate kernel, up to four wavefronts of 32 rows per
    // workgroup, at most kMaxChunks key chunks.
    c->g_waves = n_g <= 32 ? 1 : (n_g <= 64 ? 2 : 4);
    const int rows_per_set = c->g_waves * kWaveRows;
    c->g_rows = rows_per_set;
    c->n_sets = (n_g + rows_per_set - 1) / rows_per_set;
    const long long bhs = (long long)B * H * c->n_sets;
    const int tiles = (N + kTileKeys - 1) / kTileKeys;
    const int max_chunks = std::min(kMaxChunks, tiles);
    int chunks = (int)std::min<long long>(max_chunks, (kGlobTarget + bhs - 1) / bhs);
    chunks = std::max(1, chunks);
    int per = (N + chunks - 1) / chunks;
    per = (per + kTileKeys - 1) / kTileKeys * kTileKeys;
    c->chunk_keys = per;
    c->n_chunks = (N + per - 1) / per;
    c->n_glob_wg = (int)(bhs * c->n_chunks);
  }
  if (table.size() > (size_t)INT32_MAX) { free_ctx(c); return LFATTN_EUNSUPPORTED; }
  c->n_band_wg = (int)table.size();

  // ---- device state ----
  lfattn_status st = LFATTN_OK;
  if (hipGetDevice(&c->device) != hipSuccess) { free_ctx(c); return LFATTN_EHIP; }
  if ((st = dev_alloc(&c->d_work, table.size())) != LFATTN_OK ||
      (st = dev_alloc(&c->d_isglob, (size_t)N)) != LFATTN_OK ||
      (st = dev_alloc(&c->d_glob, (size_t)std::max(n_g, 1))) != LFATTN_OK) {
    free_ctx(c);
    return st;
  }
  if (n_g > 0) {
    const size_t rec = (size_t)D + 4;
    const size_t n_part = (size_t)B * H * c->n_sets * c->n_chunks * c->g_rows * rec;
    if ((st = dev_alloc(&c->d_part, n_part)) != LFATTN_OK) {
      free_ctx(c);
      return st;
    }
  }
  bool ok = hipMemcpy(c->d_work, table.data(), table.size() * sizeof(BandWork),
                      hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMemcpy(c->d_isglob, isg.data(), N, hipMemcpyHostToDevice) == hipSuccess;
  if (n_g > 0) {
    ok = ok && hipMemcpy(c->d_glob, c->glob.data(), n_g * sizeof(int), hipMemcpyHostToDevice) == hipSuccess;
  }
  if (!ok) {
    (void)hipGetLastError();
    free_ctx(c);
    return LFATTN_EHIP;
  }
  *out = c;
  return LFATTN_OK;
}

lfattn_status lfattn_forward(lfattn_t c, const void* Q, const void* K, const void* V, void* O,
                             hipStream_t stream) {
  if (!c || !Q || !K || !V || !O) return LFATTN_EINVAL;
  const uintptr_t mis = ((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u;
  if (mis) return LFATTN_EINVAL;
  const size_t bytes = (size_t)c->B * c->H * c->N * c->D * (c->dtype == LFATTN_BF16 ? 2 : 4);
  if (overlaps(O, Q, bytes) || overlaps(O, K, bytes) || overlaps(O, V, bytes)) return LFATTN_EINVAL;

  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != c->device) return LFATTN_EINVAL;

  const float sl2 = c->scale * 1.4426950408889634f;
  const bool timed = c->timing && c->n_timed < kMaxTimedForwards;
  hipEvent_t* ev = timed ? &c->ev[kEvPerForward * c->n_timed] : nullptr;
  lfattn::Timing t_band, t_part, t_merge;
  if (timed) {
    t_band = {ev[0], ev[1]};
    t_part = {ev[2], ev[3]};
    t_merge = {ev[4], ev[5]};
  }

  // Global rows: partials first, then the band kernel, then the merge (which
  // reads the partials after the kernel boundary made them visible).
  const int n_g = (int)c->glob.size();
  lfattn::GlobArgs g;
  if (n_g > 0) {
    g.Q = Q; g.K = K; g.V = V; g.O = O;
    g.glob = c->d_glob; g.part = c->d_part;
    g.H = c->H; g.N = c->N; g.n_glob = n_g; g.n_bh = c->B * c->H;
    g.rows_per_set = c->g_rows;
    g.n_sets = c->n_sets; g.n_chunks = c->n_chunks; g.chunk_keys = c->chunk_keys;
    g.sl2 = sl2;
    if (!c->glob_items &&
        lfattn::launch_glob(c->dtype, c->D, c->g_waves, g, c->n_glob_wg, stream, t_part) != hipSuccess)
      return LFATTN_EHIP;
  }

  lfattn::BandArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O;
  a.work = c->d_work; a.glob = c->d_glob; a.is_glob = c->d_isglob;
  a.H = c->H; a.N = c->N; a.hw = c->hw; a.n_glob = n_g; a.sl2 = sl2;
  a.rows_per_wg = c->band_rows;
  a.part = c->glob_items ? c->d_part : nullptr;
  a.n_sets = c->n_sets; a.n_chunks = c->n_chunks; a.chunk_keys = c->chunk_keys;
  if (lfattn::launch_band(c->dtype, c->D, a, c->n_band_wg, stream, t_band) != hipSuccess)
    return LFATTN_EHIP;

  if (n_g > 0 && lfattn::launch_glob_merge(c->dtype, c->D, g, stream, t_merge) != hipSuccess)
    return LFATTN_EHIP;

  if (timed) ++c->n_timed;
  return LFATTN_OK;
}

lfattn_status lfattn_destroy(lfattn_t c) {
  if (!c) return LFATTN_OK;
  (void)hipDeviceSynchronize();
  free_ctx(c);
  return LFATTN_OK;
}

lfattn_status lfattn_scored_pairs(lfattn_t c, long long* pairs) {
  if (!c || !pairs) return LFATTN_EINVAL;
  *pairs = c->pairs;
  return LFATTN_OK;
}

lfattn_status lfattn_band_launch_pairs(lfattn_t c, long long* pairs) {
  if (!c || !pairs) return LFATTN_EINVAL;
  const long long glob_rows = (long long)c->B * c->H * (long long)c->glob.size() * c->N;
  *pairs = c->glob_items ? c->pairs : c->pairs - glob_rows;
  return LFATTN_OK;
}

lfattn_status lfattn_band_rows(lfattn_t c, int* rows) {
  if (!c || !rows) return LFATTN_EINVAL;
  *rows = c->band_rows;
  return LFATTN_OK;
}

lfattn_status lfattn_global_list(lfattn_t c, int* out, int capacity, int* n_out) {
  if (!c || !n_out || capacity < 0 || (capacity > 0 && !out)) return LFATTN_EINVAL;
  const int n = (int)c->glob.size();
  for (int t = 0; t < n && t < capacity; ++t) out[t] = c->glob[t];
  *n_out = n;
  return LFATTN_OK;
}

lfattn_status lfattn_set_timing(lfattn_t c, int enable) {
  if (!c) return LFATTN_EINVAL;
  if (enable && c->ev.empty()) {
    c->ev.resize(kEvPerForward * kMaxTimedForwards, nullptr);
    for (auto& e : c->ev)
      if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        for (auto& x : c->ev)
          if (x) (void)hipEventDestroy(x);
        c->ev.clear();
        return LFATTN_EHIP;
      }
  }
  c->timing = enable != 0;
  c->n_timed = 0;
  return LFATTN_OK;
}

lfattn_status lfattn_read_timing(lfattn_t c, double* band_ms, double* global_ms, int* n_forwards) {
  if (!c || !band_ms || !global_ms || !n_forwards) return LFATTN_EINVAL;
  double b = 0.0, g = 0.0;
  const bool has_glob = !c->glob.empty();
  if (c->n_timed > 0) {
    hipEvent_t* last = &c->ev[kEvPerForward * (c->n_timed - 1)];
    if (hipEventSynchronize(last[has_glob ? 5 : 1]) != hipSuccess) return LFATTN_EHIP;
  }
  for (int t = 0; t < c->n_timed; ++t) {
    hipEvent_t* e = &c->ev[kEvPerForward * t];
    float x = 0.0f, y = 0.0f, z = 0.0f;
    if (hipEventElapsedTime(&x, e[0], e[1]) != hipSuccess) return LFATTN_EHIP;
    if (has_glob && !c->glob_items && hipEventElapsedTime(&y, e[2], e[3]) != hipSuccess)
      return LFATTN_EHIP;
    if (has_glob && hipEventElapsedTime(&z, e[4], e[5]) != hipSuccess) return LFATTN_EHIP;
    b += x;
    g += y + z;
  }
  *band_ms = b;
  *global_ms = g;
  *n_forwards = c->n_timed;
  c->n_timed = 0;
  return LFATTN_OK;
}

}  // extern "C"
