// C-ABI entry points of liblfattn (declared in include/lfattn.h): argument
// checks, the canonical global list, the band work table, workspace, and the
// kernel launches.
#include "lfattn.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
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
// ... and per backward: rows, keys and merge kernels, start/stop each.
constexpr int kMaxTimedBackwards = 1024;
constexpr int kEvPerBackward = 6;
constexpr int kXcds = 8;           // MI355X: workgroups go round-robin over 8 XCDs
constexpr int kMaxChunks = lfattn::kMergeBatch;  // key chunks per global row set
constexpr int kGlobTarget = 1024;  // aim for this many global-row workgroups
// Keys per global-row item of the band launch: short items when the whole
// launch fits one round of workgroup slots (they then set the critical
// path), longer ones otherwise (fewer items, less per-item overhead).
constexpr int kGlobItemKeysShort = 256, kGlobItemKeysLong = 512;
// ... and longer still when they are spread among the band items of a long
// launch (kSpreadRounds): fewer items, partial records and merge reads.
constexpr int kGlobItemKeysSpread = 1024;
constexpr int kWideRounds = 2;
// From this many rounds of band items per round of workgroup slots on, the
// global-row items are spread evenly among the band items instead of
// following them: in a long launch they would otherwise form a last phase of
// their own, bound by their memory traffic, while spread out they overlap the
// band items' arithmetic.  (In a launch of one or two rounds, dispatching them
// last measured faster.)
constexpr int kSpreadRounds = 4;
// Backward work items: rows or keys per item, and the key or row chunk of a
// global item.
constexpr int kBwdChunk = 512, kBwdChunkShort = 256;
constexpr int kBwdShortRounds = 2;
// At most this many chunks per global set (longer chunks past 32768 keys),
// bounding the partial-gradient workspace.
constexpr int kBwdMaxChunks = 64;
constexpr long long kMaxN = 1LL << 29;

// Static scratch of lfattn_forward_noalloc: the global-row partial records
// of calls that may not allocate.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` only names the symbol:
// kernels take the per-device address from scratch_ptr(), never the name.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
// Its layout: the global-row sets' arrival counts (zero between calls),
// then the partial records.
constexpr size_t kScratchCounts = 65536;
constexpr size_t kScratchPartOffset = kScratchCounts * sizeof(unsigned);

// Device address of `scratch` per device ordinal, looked up once per device
// (hipGetSymbolAddress with that device current) by the first lfattn_create
// on it; nullptr until then or when the lookup failed.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_tried[kMaxDevices] = {};

void scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_tried[dev]) return;
  g_scratch_tried[dev] = true;
  void* p = nullptr;
  // The arrival counts start at zero (each call leaves them at zero).
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr &&
      hipMemset(p, 0, kScratchPartOffset) == hipSuccess) {
    g_scratch_ptr[dev] = p;
  } else {
    (void)hipGetLastError();
  }
}

void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[dev];
}

}  // namespace

struct lfattn_ctx {
  int B = 0, H = 0, N = 0, D = 0, dtype = 0, window = 0, hw = 0;
  bool causal = false;  // the band's left half and the row itself
  int chunk = 0;        // > 0: chunked attention with chunks of this length
  int n_memory = 0;     // chunked: memory positions 0 .. n_memory - 1 (the global rows)
  float scale = 0.0f;
  std::vector<int> dil;
  // Global lists, sorted and without repeats: gl[0] for every batch element
  // (shared), or gl[b] for batch element b.
  std::vector<std::vector<int>> gl;
  bool shared = true;
  int n_gmax = 0;  // the longest list
  long long n_gsum = 0;  // sum over the batch of the list lengths
  const std::vector<int>& G(int b) const { return gl[shared ? 0 : b]; }
  long long pairs = 0;
  int device = 0;

  BandWork* d_work = nullptr;
  // Backward pass (bf16, D = 64): its work table and the per-row Delta.
  BandWork* d_bwork = nullptr;  // backward tables: row side, then key side
  int n_bwork[2] = {0, 0};
  float* d_terms = nullptr;  // backward: the key side's per-row terms (three planes)
  float* d_gpart = nullptr;  // backward: global items' partial gradients
  int n_gch = 0;             // backward: key (row) chunks of a global item
  int n_band_wg = 0;
  int* d_glob = nullptr;           // the distinct lists, one after another
  int2* d_gsel = nullptr;          // [B]: (offset, length) of each batch element's list
  unsigned char* d_isglob = nullptr;  // [1 or B][N]

  float* d_part = nullptr;
  size_t part_bytes = 0;  // bytes of the global-row partial records
  unsigned* d_gcount = nullptr;  // arrival count per (b*H + h, set) of the fused merge
  size_t n_gcount = 0;
  int band_rows = 0;  // rows per band workgroup
  int bwd_rows[2] = {0, 0};  // rows (keys) per backward item, row / key side: 64 or 128
  int bwd_rows_wpe = 0;      // query side, D = 64: its kernel's wavefronts per SIMD (3 or 4)
  int bwd_chunk = 0;  // keys (rows) per chunk of a backward global item
  int g_waves = 0, g_rows = 0, n_sets = 0, n_chunks = 0, chunk_keys = 0, n_glob_wg = 0;
  bool glob_items = false;  // global-row partials run as items of the band launch
  bool fuse_merge = false;  // ... and the band launch merges them too
  bool one_round = false;   // the band launch fits one round of workgroup slots

  // Device memory comes from the stream-ordered allocator on this private
  // stream (async_mem), so that lfattn_destroy can release it behind the
  // stream of the handle's latest call (`last`, an event recorded there at
  // destroy) without waiting for the whole device.
  hipStream_t mem_stream = nullptr;
  bool async_mem = false;
  hipEvent_t done = nullptr;
  hipStream_t last = nullptr;
  bool used = false;

  bool timing = false;
  int n_timed = 0;
  std::vector<hipEvent_t> ev;  // kEvPerForward per timed forward
  int n_btimed = 0;
  std::vector<hipEvent_t> bev;  // kEvPerBackward per timed backward
};

namespace {

template <typename T>
lfattn_status dev_alloc(lfattn_ctx* c, T** p, size_t count) {
  *p = nullptr;
  if (count == 0) return LFATTN_OK;
  const hipError_t e = c->async_mem ? hipMallocAsync((void**)p, count * sizeof(T), c->mem_stream)
                                    : hipMalloc((void**)p, count * sizeof(T));
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return LFATTN_ENOMEM;
  }
  return LFATTN_OK;
}

// Whether work enqueued on `stream` is being captured into a graph.
bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return cs != hipStreamCaptureStatusNone;
}

// Release a handle: its device memory goes back behind the work enqueued so
// far on the stream of its latest call (stream-ordered frees after an event
// recorded there), without a device-wide wait.  Where that cannot be ordered
// (the event cannot be recorded), the device is waited for first.  With the
// plain allocator (no memory pools) hipFree itself waits for the device.
void free_ctx(lfattn_ctx* c) {
  if (!c) return;
  void* ptrs[] = {c->d_work, c->d_glob, c->d_gsel, c->d_isglob, c->d_part, c->d_bwork,
                  c->d_terms, c->d_gpart, c->d_gcount};
  if (c->async_mem) {
    if (c->used && !capturing(c->last)) {
      if (hipEventRecord(c->done, c->last) != hipSuccess ||
          hipStreamWaitEvent(c->mem_stream, c->done, 0) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipDeviceSynchronize();
      }
    }
    for (void* p : ptrs)
      if (p) (void)hipFreeAsync(p, c->mem_stream);
  } else {
    for (void* p : ptrs)
      if (p) (void)hipFree(p);
  }
  if (c->done) (void)hipEventDestroy(c->done);
  for (hipEvent_t e : c->ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->bev) (void)hipEventDestroy(e);
  if (c->mem_stream) (void)hipStreamDestroy(c->mem_stream);
  (void)hipGetLastError();
  delete c;
}


// Scored pairs of one head with dilation d: every row's band (keys i + d*k,
// |k| <= hw, inside [0, N); causal: -hw <= k <= 0), plus the global keys
// outside that band; global rows score all N keys.  chunk > 0: a row past the
// memory scores its chunk and the memory.
long long head_pairs(int N, long long hw, int d, bool causal, int chunk, int n_memory,
                     const std::vector<int>& glob, const std::vector<unsigned char>& isg) {
  long long total = 0;
  for (long long i = 0; i < N; ++i) {
    if (isg[i]) {
      total += N;
      continue;
    }
    if (chunk > 0) {
      const long long c0 = n_memory + (i - n_memory) / chunk * chunk;
      total += std::min<long long>(c0 + chunk, N) - c0 + n_memory;
      continue;
    }
    long long left = std::min(i / d, hw), right = causal ? 0 : std::min((N - 1 - i) / d, hw);
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

lfattn_status forward_impl(lfattn_t c, const void* Q, const void* K, const void* V,
                           const void* Qg, const void* Kg, const void* Vg, void* O, float* lse,
                           hipStream_t stream, float* part, unsigned* counts);

bool overlaps(const void* a, const void* b, size_t bytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bytes && y < x + bytes;
}

// Whether [a, a + abytes) and [b, b + bbytes) share a byte.
bool overlaps2(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bbytes && y < x + abytes;
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
    case LFATTN_ESCRATCH: return "needs more than the static scratch array";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

// Shared checks of the create entry points (no HIP call).
lfattn_status check_shape(int B, int H, int N, int D, lfattn_dtype dtype, int window,
                          const int* dilation, float scale) {
  if (B < 1 || H < 1 || N < 1 || D < 1 || window < 0) return LFATTN_EINVAL;
  if (dtype != LFATTN_F32 && dtype != LFATTN_BF16) return LFATTN_EINVAL;
  if (std::isnan(scale) || std::isinf(scale)) return LFATTN_EINVAL;
  if (dilation)
    for (int h = 0; h < H; ++h)
      if (dilation[h] < 1) return LFATTN_EINVAL;
  return LFATTN_OK;
}

lfattn_status check_support(int B, int H, int N, int D) {
  if (D != 64 && D != 128) return LFATTN_EUNSUPPORTED;
  if ((long long)N >= kMaxN || (long long)B * H > (1LL << 24)) return LFATTN_EUNSUPPORTED;
  return LFATTN_OK;
}

// The handle, once the arguments are checked: gl holds one canonical list
// (shared) or one per batch element.
lfattn_status create_impl(lfattn_t* out, int B, int H, int N, int D, lfattn_dtype dtype,
                          int window, const int* dilation,
                          std::vector<std::vector<int>>&& gl, bool shared, bool causal,
                          int chunk, float scale) {
  lfattn_ctx* c = new (std::nothrow) lfattn_ctx;
  if (!c) return LFATTN_ENOMEM;
  c->B = B; c->H = H; c->N = N; c->D = D; c->dtype = (int)dtype; c->window = window;
  c->causal = causal;
  c->chunk = chunk;
  c->n_memory = chunk > 0 ? (int)gl[0].size() : 0;  // chunked: G = {0 .. M-1}
  c->hw = (int)std::min<long long>(window / 2, N);  // a wider half-width changes nothing
  c->scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
  c->dil.assign(H, 1);
  if (dilation) c->dil.assign(dilation, dilation + H);
  c->gl = std::move(gl);
  c->shared = shared;
  for (int b = 0; b < B; ++b) {
    c->n_gmax = std::max(c->n_gmax, (int)c->G(b).size());
    c->n_gsum += (long long)c->G(b).size();
  }
  if (dtype == LFATTN_BF16 && c->n_gmax > lfattn::kMaxGlobalBf16) {
    delete c;
    return LFATTN_EUNSUPPORTED;
  }
  const int n_lists = (int)c->gl.size();
  std::vector<unsigned char> isg((size_t)n_lists * N, 0);
  for (int t = 0; t < n_lists; ++t)
    for (int g : c->gl[t]) isg[(size_t)t * N + g] = 1;

  // Scored pairs, per list and distinct dilation value.
  {
    std::vector<int> ds = c->dil;
    std::sort(ds.begin(), ds.end());
    ds.erase(std::unique(ds.begin(), ds.end()), ds.end());
    c->pairs = 0;
    for (int t = 0; t < n_lists; ++t) {
      const std::vector<unsigned char> row(isg.begin() + (size_t)t * N,
                                           isg.begin() + (size_t)(t + 1) * N);
      long long total = 0;
      for (int d : ds) {
        long long per =
            head_pairs(N, window / 2, d, causal, chunk, c->n_memory, c->gl[t], row);
        total += per * (long long)std::count(c->dil.begin(), c->dil.end(), d);
      }
      c->pairs += total * (shared ? B : 1);
    }
  }
  // Offset and length of each batch element's list in the device array.
  std::vector<int> goff(n_lists + 1, 0);
  for (int t = 0; t < n_lists; ++t) goff[t + 1] = goff[t] + (int)c->gl[t].size();
  std::vector<int2> gsel(B);
  for (int b = 0; b < B; ++b) {
    const int t = shared ? 0 : b;
    gsel[b] = make_int2(goff[t], goff[t + 1] - goff[t]);
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

  // Rows (keys) per backward item: 64 on both sides (each workgroup's tiles
  // split between two pairs of wavefronts: twice the workgroups of 128-row
  // items, whose one tile stream four 32-row blocks share), the faster choice
  // on every bf16 workload measured; LFATTN_BWD_ROWS=64 or 128 sets both (both
  // give the same results; this lets the tests run every kernel).
  if (dtype == LFATTN_BF16) {
    c->bwd_rows[0] = 64;
    c->bwd_rows[1] = 64;
    if (const char* e = std::getenv("LFATTN_BWD_ROWS")) {
      if (std::strcmp(e, "64") == 0) c->bwd_rows[0] = c->bwd_rows[1] = 64;
      if (std::strcmp(e, "128") == 0) c->bwd_rows[0] = c->bwd_rows[1] = 128;
    }
  }

  // Band work: one item per workgroup's rows of each (b, h, residue r)
  // subsequence, laid out so that the items the hardware sends to one XCD
  // (blockIdx congruent mod 8) are consecutive query blocks of the same head,
  // which share their band's K and V rows in that XCD's L2.
  std::vector<BandWork> items;
  for (int bh = 0; bh < B * H; ++bh) {
    const int d = c->dil[bh % H], b = bh / H;
    for (int r = 0; r < d && r < N; ++r) {
      const int Lr = (N - r + d - 1) / d;
      for (int t0 = 0; t0 < Lr; t0 += band_rows)
        items.push_back(BandWork{bh, r, t0, d, gsel[b].x, gsel[b].y, b, 0});
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
  // item of the band launch, after the band items, so that those workgroups
  // are dispatched last and fill the slots the band items leave free (in a
  // launch of many rounds, spread among them: kSpreadRounds).  fp32: a
  // separate kernel (below).
  // (Sets are counted per batch element; records are laid out for the
  // longest list.)
  const int n_g = c->n_gmax;
  c->glob_items = n_g > 0 && lfattn::band_takes_global_items(dtype, D);
  if (c->glob_items) {
    c->g_rows = lfattn::global_set_rows(D, band_rows);  // rows of G per global item
    c->n_sets = (n_g + c->g_rows - 1) / c->g_rows;
    long long set_count = 0;  // sum over (b, h) of the row sets
    for (int b = 0; b < B; ++b)
      set_count += (long long)H * ((gsel[b].y + c->g_rows - 1) / c->g_rows);
    const long long short_items =
        set_count * ((N + kGlobItemKeysShort - 1) / kGlobItemKeysShort);
    int keys = n_items + short_items <= slots ? kGlobItemKeysShort
               : (long long)n_items >= kSpreadRounds * slots ? kGlobItemKeysSpread
                                                             : kGlobItemKeysLong;
    // The band launch can merge the global rows itself (the last chunk item
    // of a set to finish merges it; chunks long enough that a set has at most
    // kFuseChunks of them).  It measured slower than the separate merge
    // launch on these workloads (the records cross XCDs through device-
    // coherent accesses, 3 us to write and 1.5 us per round of reads), so it
    // is taken only when LFATTN_FUSE_MERGE=1 at create.
    c->fuse_merge = false;
    if (const char* e = std::getenv("LFATTN_FUSE_MERGE")) c->fuse_merge = std::strcmp(e, "1") == 0;
    if (c->fuse_merge) {
      const int min_keys = (N + lfattn::kFuseChunks - 1) / lfattn::kFuseChunks;
      keys = std::max(keys, (min_keys + 31) / 32 * 32);
    }
    c->chunk_keys = keys;
    c->n_chunks = (N + keys - 1) / keys;
    // Each global item goes to the XCD of the residue-0 band item whose rows
    // start nearest its chunk (that XCD's L2 holds the chunk's K and V rows):
    // items are queued per XCD.
    std::vector<std::vector<BandWork>> q(kXcds);
    std::vector<int> first_item(B * H, -1);
    for (int k = 0; k < n_items; ++k)
      if (first_item[items[k].bh] < 0) first_item[items[k].bh] = k;
    for (int bh = 0; bh < B * H; ++bh) {
      const int b = bh / H;
      const int sets_b = (gsel[b].y + c->g_rows - 1) / c->g_rows;
      for (int set = 0; set < sets_b; ++set)
        for (int ch = 0; ch < c->n_chunks; ++ch) {
          const int d = c->dil[bh % H];
          const long long key0 = (long long)ch * keys;
          // residue 0's items come first for this head; its subsequence
          // position of key0 is key0 / d.
          const int k = std::min(first_item[bh] + (int)(key0 / d / band_rows), n_items - 1);
          q[item_xcd[std::max(k, 0)]].push_back(
              BandWork{bh, set, ch, 0, gsel[b].x, gsel[b].y, b, 0});
        }
    }
    // Per XCD, the order of its items: each head's global items right after
    // that head's last band item there (its K and V rows are then still in
    // the XCD's L2: at 16K tokens this cuts the band launch's HBM reads by
    // 12%), or (long launches) each global item at its proportional place.
    std::vector<std::vector<BandWork>> ml(kXcds);
    const bool spread = (long long)n_items >= kSpreadRounds * slots;
    {
      std::vector<std::vector<BandWork>> bl(kXcds);
      for (int bid = 0; bid < n_items; ++bid) bl[bid % kXcds].push_back(table[bid]);
      for (int x = 0; x < kXcds && !spread; ++x) {
        std::vector<char> used(q[x].size(), 0);
        for (size_t ib = 0; ib < bl[x].size(); ++ib) {
          ml[x].push_back(bl[x][ib]);
          const int bh = bl[x][ib].bh;
          if (ib + 1 < bl[x].size() && bl[x][ib + 1].bh == bh) continue;
          for (size_t ig = 0; ig < q[x].size(); ++ig)
            if (!used[ig] && q[x][ig].bh == bh) {
              ml[x].push_back(q[x][ig]);
              used[ig] = 1;
            }
        }
        for (size_t ig = 0; ig < q[x].size(); ++ig)
          if (!used[ig]) ml[x].push_back(q[x][ig]);
      }
      for (int x = 0; x < kXcds && spread; ++x) {
        const size_t nb = bl[x].size(), ng = q[x].size(), tot = nb + ng;
        size_t ib = 0, ig = 0;
        for (size_t k2 = 0; k2 < tot; ++k2) {
          const bool take_g = ig < ng && (ib >= nb || k2 * ng >= (2 * ig + 1) * tot / 2);
          ml[x].push_back(take_g ? q[x][ig++] : bl[x][ib++]);
        }
      }
    }
    // Block indices congruent to x (mod 8) run on XCD x: deal each list to
    // them in order, falling back to another list when one runs dry.
    table.clear();
    size_t left = 0;
    for (auto& v : ml) left += v.size();
    std::vector<size_t> pos(kXcds, 0);
    while (left > 0) {
      int x = (int)(table.size() % kXcds);
      for (int t = 0; t < kXcds && pos[x] >= ml[x].size(); ++t) x = (x + 1) % kXcds;
      table.push_back(ml[x][pos[x]++]);
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
  c->one_round = (long long)c->n_band_wg <= slots;

  // Backward work (bf16, D = 64), one table per side: band items of
  // bwd_rows rows (row side) or keys (key side) per (b, h, residue), then
  // items of bwd_rows global positions against a chunk of bwd_chunk keys
  // (row side) or rows (key side).
  std::vector<BandWork> btable;
  const bool has_bwd = dtype == LFATTN_BF16;
  if (has_bwd) {
    // Chunks of kBwdChunkShort keys (rows) when a side's band items and global
    // items come to less than kBwdShortRounds rounds of workgroup slots: the
    // global items, dispatched last, then form a short tail; kBwdChunk
    // otherwise (fewer partials to merge).
    int chunk = kBwdChunk;
    if (n_g > 0) {
      long long n_band_items = 0;
      for (int bh = 0; bh < B * H; ++bh) {
        const int d = c->dil[bh % H];
        for (int r = 0; r < d && r < N; ++r)
          n_band_items += ((N - r + d - 1) / d + c->bwd_rows[0] - 1) / c->bwd_rows[0];
      }
      long long sets = 0;
      for (int b = 0; b < B; ++b) sets += (long long)H * ((gsel[b].y + c->bwd_rows[0] - 1) / c->bwd_rows[0]);
      const long long bwd_slots = (long long)(D == 64 ? 3 : 2) * cus;
      if (n_band_items + sets * ((N + kBwdChunk - 1) / kBwdChunk) < kBwdShortRounds * bwd_slots)
        chunk = kBwdChunkShort;
    }
    c->bwd_chunk = std::max(chunk, (N + kBwdMaxChunks * 32 - 1) / (kBwdMaxChunks * 32) * 32);
    c->n_gch = (N + c->bwd_chunk - 1) / c->bwd_chunk;
    for (int side = 0; side < 2; ++side) {
      const int rows = c->bwd_rows[side];
      const size_t start = btable.size();
      for (int bh = 0; bh < B * H; ++bh) {
        const int d = c->dil[bh % H], b = bh / H;
        for (int r = 0; r < d && r < N; ++r) {
          const int Lr = (N - r + d - 1) / d;
          for (int t0 = 0; t0 < Lr; t0 += rows)
            btable.push_back(BandWork{bh, r, t0, d, gsel[b].x, gsel[b].y, b, 0});
        }
      }
      const size_t gstart = btable.size();
      for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H;
        const int sets_b = (gsel[b].y + rows - 1) / rows;
        for (int set = 0; set < sets_b; ++set)
          for (int ch = 0; ch < c->n_gch; ++ch)
            btable.push_back(BandWork{bh, set, ch, 0, gsel[b].x, gsel[b].y, b, 0});
      }
      if (btable.size() - start > (size_t)INT32_MAX) { free_ctx(c); return LFATTN_EUNSUPPORTED; }
      c->n_bwork[side] = (int)(btable.size() - start);
      // Block indices congruent to x (mod 8) run on XCD x: each XCD takes a
      // run of consecutive band items (which share their neighbours' row or
      // key tiles in that XCD's L2), then its share of the global items.
      {
        std::vector<std::vector<BandWork>> ml(kXcds);
        for (const size_t lo0 : {start, gstart}) {
          const size_t hi0 = lo0 == start ? gstart : btable.size(), n = hi0 - lo0;
          for (int x = 0; x < kXcds; ++x)
            ml[x].insert(ml[x].end(), btable.begin() + lo0 + n * x / kXcds,
                         btable.begin() + lo0 + n * (x + 1) / kXcds);
        }
        std::vector<size_t> pos(kXcds, 0);
        for (size_t bid = 0; bid < btable.size() - start; ++bid) {
          int x = (int)(bid % kXcds);
          for (int t = 0; t < kXcds && pos[x] >= ml[x].size(); ++t) x = (x + 1) % kXcds;
          btable[start + bid] = ml[x][pos[x]++];
        }
      }
    }
    // The query side at D = 64 runs at four wavefronts per SIMD (a third more
    // workgroups per round, with a leaner register budget) when its items
    // come to two or more rounds of three-per-CU slots: 8K -6%, 16K -7%; at
    // Longformer-base (1.25 rounds) three are faster.  LFATTN_BWD_ROWS_WPE=3
    // or 4 overrides the choice (both give the same results).
    c->bwd_rows_wpe = 3;
    if (D == 64 && (long long)c->n_bwork[0] >= 2LL * 3 * cus) c->bwd_rows_wpe = 4;
    if (D == 64)
      if (const char* e = std::getenv("LFATTN_BWD_ROWS_WPE")) {
        if (std::strcmp(e, "3") == 0) c->bwd_rows_wpe = 3;
        if (std::strcmp(e, "4") == 0) c->bwd_rows_wpe = 4;
      }
  }

  // ---- device state ----
  lfattn_status st = LFATTN_OK;
  if (hipGetDevice(&c->device) != hipSuccess) { free_ctx(c); return LFATTN_EHIP; }
  if (hipStreamCreateWithFlags(&c->mem_stream, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&c->done, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    free_ctx(c);
    return LFATTN_EHIP;
  }
  {
    int pools = 0;
    c->async_mem = hipDeviceGetAttribute(&pools, hipDeviceAttributeMemoryPoolsSupported,
                                         c->device) == hipSuccess && pools != 0;
    (void)hipGetLastError();
  }
  if ((st = dev_alloc(c, &c->d_work, table.size())) != LFATTN_OK ||
      (st = dev_alloc(c, &c->d_isglob, isg.size())) != LFATTN_OK ||
      (st = dev_alloc(c, &c->d_glob, (size_t)std::max(goff[n_lists], 1))) != LFATTN_OK ||
      (st = dev_alloc(c, &c->d_gsel, (size_t)B)) != LFATTN_OK) {
    free_ctx(c);
    return st;
  }
  if (has_bwd && ((st = dev_alloc(c, &c->d_bwork, btable.size())) != LFATTN_OK ||
                   (st = dev_alloc(c, &c->d_terms, (size_t)3 * B * H * N)) != LFATTN_OK ||
                   (n_g > 0 &&
                    (st = dev_alloc(c, &c->d_gpart, (size_t)3 * B * H * c->n_gch * n_g * D)) !=
                        LFATTN_OK))) {
    free_ctx(c);
    return st;
  }
  if (n_g > 0) {
    const size_t rec = (size_t)D + 4;
    const size_t n_part = (size_t)B * H * c->n_sets * c->n_chunks * c->g_rows * rec;
    c->part_bytes = n_part * sizeof(float);
    if ((st = dev_alloc(c, &c->d_part, n_part)) != LFATTN_OK) {
      free_ctx(c);
      return st;
    }
    if (c->fuse_merge) {
      c->n_gcount = (size_t)B * H * c->n_sets;
      if ((st = dev_alloc(c, &c->d_gcount, c->n_gcount)) != LFATTN_OK) {
        free_ctx(c);
        return st;
      }
      if (hipMemsetAsync(c->d_gcount, 0, c->n_gcount * sizeof(unsigned), c->mem_stream) !=
          hipSuccess) {
        (void)hipGetLastError();
        free_ctx(c);
        return LFATTN_EHIP;
      }
    }
  }
  scratch_setup(c->device);
  std::vector<int> flat;
  for (const auto& v : c->gl) flat.insert(flat.end(), v.begin(), v.end());
  auto up = [&](void* dst, const void* src, size_t bytes) {
    return bytes == 0 ||
           hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, c->mem_stream) == hipSuccess;
  };
  bool ok = up(c->d_work, table.data(), table.size() * sizeof(BandWork));
  ok = ok && up(c->d_isglob, isg.data(), isg.size());
  if (has_bwd) ok = ok && up(c->d_bwork, btable.data(), btable.size() * sizeof(BandWork));
  ok = ok && up(c->d_gsel, gsel.data(), B * sizeof(int2));
  ok = ok && up(c->d_glob, flat.data(), flat.size() * sizeof(int));
  // The tables are in place (and the host vectors may go) before any call.
  ok = ok && hipStreamSynchronize(c->mem_stream) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    free_ctx(c);
    return LFATTN_EHIP;
  }
  *out = c;
  return LFATTN_OK;
}

}  // namespace

extern "C" {

lfattn_status lfattn_create(lfattn_t* out, int B, int H, int N, int D, lfattn_dtype dtype,
                            int window, const int* dilation, const int* global_idx,
                            int n_global, float scale) {
  // ---- argument checks: no HIP call before all of them pass ----
  if (!out) return LFATTN_EINVAL;
  *out = nullptr;
  lfattn_status st = check_shape(B, H, N, D, dtype, window, dilation, scale);
  if (st != LFATTN_OK) return st;
  if (n_global < 0 || (n_global > 0 && !global_idx)) return LFATTN_EINVAL;
  for (int t = 0; t < n_global; ++t)
    if (global_idx[t] < 0 || global_idx[t] >= N) return LFATTN_EINVAL;
  if ((st = check_support(B, H, N, D)) != LFATTN_OK) return st;
  // Canonical global list: sorted, repeats removed (a position listed twice is
  // global once, as setting a mask row or column twice changes nothing).
  std::vector<std::vector<int>> gl(1);
  gl[0].assign(global_idx, global_idx + n_global);
  std::sort(gl[0].begin(), gl[0].end());
  gl[0].erase(std::unique(gl[0].begin(), gl[0].end()), gl[0].end());
  return create_impl(out, B, H, N, D, dtype, window, dilation, std::move(gl), true, false, 0,
                     scale);
}

lfattn_status lfattn_create_chunked(lfattn_t* out, int B, int H, int N, int D,
                                    lfattn_dtype dtype, int chunk, int n_memory, float scale) {
  if (!out) return LFATTN_EINVAL;
  *out = nullptr;
  lfattn_status st = check_shape(B, H, N, D, dtype, 0, nullptr, scale);
  if (st != LFATTN_OK) return st;
  if (chunk < 1 || n_memory < 0 || n_memory > N) return LFATTN_EINVAL;
  if ((st = check_support(B, H, N, D)) != LFATTN_OK) return st;
  // The memory tokens are the global positions 0 .. M-1.
  std::vector<std::vector<int>> gl(1);
  for (int m = 0; m < n_memory; ++m) gl[0].push_back(m);
  return create_impl(out, B, H, N, D, dtype, 0, nullptr, std::move(gl), true, false, chunk,
                     scale);
}

lfattn_status lfattn_create_causal(lfattn_t* out, int B, int H, int N, int D,
                                   lfattn_dtype dtype, int window, const int* dilation,
                                   float scale) {
  if (!out) return LFATTN_EINVAL;
  *out = nullptr;
  lfattn_status st = check_shape(B, H, N, D, dtype, window, dilation, scale);
  if (st != LFATTN_OK) return st;
  if ((st = check_support(B, H, N, D)) != LFATTN_OK) return st;
  std::vector<std::vector<int>> gl(1);
  return create_impl(out, B, H, N, D, dtype, window, dilation, std::move(gl), true, true, 0,
                     scale);
}

lfattn_status lfattn_create_masked(lfattn_t* out, int B, int H, int N, int D,
                                   lfattn_dtype dtype, int window, const int* dilation,
                                   const unsigned char* global_mask, float scale) {
  if (!out) return LFATTN_EINVAL;
  *out = nullptr;
  lfattn_status st = check_shape(B, H, N, D, dtype, window, dilation, scale);
  if (st != LFATTN_OK) return st;
  if ((st = check_support(B, H, N, D)) != LFATTN_OK) return st;
  // One list per batch element, from its mask row; a single shared list when
  // every row is the same.
  std::vector<std::vector<int>> gl(B);
  if (global_mask)
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < N; ++i)
        if (global_mask[(size_t)b * N + i]) gl[b].push_back(i);
  bool shared = true;
  for (int b = 1; b < B && shared; ++b) shared = gl[b] == gl[0];
  if (shared) gl.resize(1);
  return create_impl(out, B, H, N, D, dtype, window, dilation, std::move(gl), shared, false, 0,
                     scale);
}

lfattn_status lfattn_forward(lfattn_t c, const void* Q, const void* K, const void* V, void* O,
                             hipStream_t stream) {
  return lfattn_forward_global_proj(c, Q, K, V, nullptr, nullptr, nullptr, O, stream);
}

lfattn_status lfattn_forward_global_proj(lfattn_t c, const void* Q, const void* K,
                                         const void* V, const void* Qg, const void* Kg,
                                         const void* Vg, void* O, hipStream_t stream) {
  return forward_impl(c, Q, K, V, Qg, Kg, Vg, O, nullptr, stream, c ? c->d_part : nullptr,
                      c ? c->d_gcount : nullptr);
}

lfattn_status lfattn_forward_noalloc(lfattn_t c, const void* Q, const void* K, const void* V,
                                     void* O, hipStream_t stream) {
  if (!c) return LFATTN_EINVAL;
  if (c->part_bytes > kScratchBytes - kScratchPartOffset || c->n_gcount > kScratchCounts)
    return LFATTN_ESCRATCH;
  float* part = nullptr;
  unsigned* counts = nullptr;
  if (c->part_bytes > 0) {
    unsigned char* base = (unsigned char*)scratch_ptr(c->device);
    if (!base) return LFATTN_EHIP;
    counts = (unsigned*)base;
    part = (float*)(base + kScratchPartOffset);
  }
  return forward_impl(c, Q, K, V, nullptr, nullptr, nullptr, O, nullptr, stream, part, counts);
}

lfattn_status lfattn_forward_global_proj_lse(lfattn_t c, const void* Q, const void* K,
                                             const void* V, const void* Qg, const void* Kg,
                                             const void* Vg, void* O, float* LSE,
                                             hipStream_t stream) {
  if (!c || !LSE) return LFATTN_EINVAL;
  if (c->dtype != LFATTN_BF16) return LFATTN_EUNSUPPORTED;
  // The global-row projections must not overlap the log-sum-exp either.
  const size_t bytes = (size_t)c->B * c->H * c->N * c->D * 2;
  const size_t lbytes = (size_t)c->B * c->H * c->N * sizeof(float);
  for (const void* in : {Qg, Kg, Vg})
    if (in && overlaps2(LSE, lbytes, in, bytes)) return LFATTN_EINVAL;
  return forward_impl(c, Q, K, V, Qg, Kg, Vg, O, LSE, stream, c->d_part, c->d_gcount);
}

lfattn_status lfattn_forward_lse(lfattn_t c, const void* Q, const void* K, const void* V,
                                 void* O, float* LSE, hipStream_t stream) {
  if (!c || !LSE) return LFATTN_EINVAL;
  if (c->dtype != LFATTN_BF16) return LFATTN_EUNSUPPORTED;
  return forward_impl(c, Q, K, V, nullptr, nullptr, nullptr, O, LSE, stream, c->d_part,
                      c->d_gcount);
}

}  // extern "C"

namespace {

// part, counts: where the global rows' partial records and the sets'
// arrival counts go (the handle's workspace, or the static scratch for
// lfattn_forward_noalloc).
lfattn_status forward_impl(lfattn_t c, const void* Q, const void* K, const void* V,
                           const void* Qg, const void* Kg, const void* Vg, void* O, float* lse,
                           hipStream_t stream, float* part, unsigned* counts) {
  if (!c || !Q || !K || !V || !O) return LFATTN_EINVAL;
  if (!Qg) Qg = Q;
  if (!Kg) Kg = K;
  if (!Vg) Vg = V;
  const uintptr_t mis = ((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O |
                         (uintptr_t)Qg | (uintptr_t)Kg | (uintptr_t)Vg) & 15u;
  if (mis) return LFATTN_EINVAL;
  const size_t bytes = (size_t)c->B * c->H * c->N * c->D * (c->dtype == LFATTN_BF16 ? 2 : 4);
  for (const void* in : {Q, K, V, Qg, Kg, Vg})
    if (overlaps(O, in, bytes)) return LFATTN_EINVAL;
  if (lse) {
    const size_t lbytes = (size_t)c->B * c->H * c->N * sizeof(float);
    if ((uintptr_t)lse & 3u) return LFATTN_EINVAL;
    for (const void* in : {Q, K, V, (const void*)O})
      if (overlaps2(lse, lbytes, in, bytes)) return LFATTN_EINVAL;
  }

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
  c->last = stream;
  c->used = true;

  // Global rows: partials first, then the band kernel, then the merge (which
  // reads the partials after the kernel boundary made them visible).
  const int n_g = c->n_gmax;
  lfattn::GlobArgs g;
  if (n_g > 0) {
    g.Q = Qg; g.K = Kg; g.V = Vg; g.O = O;
    g.glob = c->d_glob; g.gsel = c->d_gsel; g.part = part;
    g.H = c->H; g.N = c->N; g.n_glob = n_g; g.n_bh = c->B * c->H;
    g.rows_per_set = c->g_rows;
    g.n_sets = c->n_sets; g.n_chunks = c->n_chunks; g.chunk_keys = c->chunk_keys;
    g.sl2 = sl2;
    g.lse = lse;
    if (!c->glob_items &&
        lfattn::launch_glob(c->dtype, c->D, c->g_waves, g, c->n_glob_wg, stream, t_part) != hipSuccess)
      return LFATTN_EHIP;
  }

  lfattn::BandArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O;
  a.Qg = Qg; a.Kg = Kg; a.Vg = Vg;
  a.work = c->d_work; a.glob = c->d_glob; a.is_glob = c->d_isglob;
  a.isg_stride = c->shared ? 0 : c->N;
  a.H = c->H; a.N = c->N; a.hw = c->hw; a.n_glob = n_g; a.sl2 = sl2;
  a.hr = c->causal ? 0 : c->hw;
  a.chunk = c->chunk;
  a.lse = lse;
  a.cbase = c->n_memory;
  a.rows_per_wg = c->band_rows;
  a.part = c->glob_items ? part : nullptr;
  a.gcount = c->fuse_merge ? counts : nullptr;
  a.n_sets = c->n_sets; a.n_chunks = c->n_chunks; a.chunk_keys = c->chunk_keys;
  a.lrf = c->one_round ? 1 : 0;
  if (lfattn::launch_band(c->dtype, c->D, a, c->n_band_wg, stream, t_band) != hipSuccess)
    return LFATTN_EHIP;

  // A separate kernel merges the global rows' partials unless the band launch
  // does (fp32, and bf16 launches of several rounds of workgroup slots).
  if (n_g > 0 && !c->fuse_merge &&
      lfattn::launch_glob_merge(c->dtype, c->D, g, stream, t_merge) != hipSuccess)
    return LFATTN_EHIP;

  if (timed) ++c->n_timed;
  return LFATTN_OK;
}

// The backward pass; proj: the global rows' own projections Qg, Kg, Vg
// (NULL: Q, K, V) with their gradients in dQg, dKg, dVg.
lfattn_status backward_impl(lfattn_t c, const void* Q, const void* K, const void* V,
                            const void* Qg, const void* Kg, const void* Vg, const void* O,
                            const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                            float* dQg, float* dKg, float* dVg, bool proj, hipStream_t stream) {
  if (!c || !Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return LFATTN_EINVAL;
  if (proj && (!dQg || !dKg || !dVg)) return LFATTN_EINVAL;
  if (c->dtype != LFATTN_BF16) return LFATTN_EUNSUPPORTED;
  if (!Qg) Qg = Q;
  if (!Kg) Kg = K;
  if (!Vg) Vg = V;
  uintptr_t mis = ((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O | (uintptr_t)dO |
                   (uintptr_t)dQ | (uintptr_t)dK | (uintptr_t)dV | (uintptr_t)Qg |
                   (uintptr_t)Kg | (uintptr_t)Vg) & 15u;
  if (proj) mis |= ((uintptr_t)dQg | (uintptr_t)dKg | (uintptr_t)dVg) & 15u;
  if (mis || ((uintptr_t)LSE & 3u)) return LFATTN_EINVAL;
  const size_t n_el = (size_t)c->B * c->H * c->N * c->D;
  const size_t in_b = n_el * 2, out_b = n_el * 4, lse_b = (size_t)c->B * c->H * c->N * 4;
  // The outputs overlap no input and no other output.
  const void* outs[6] = {dQ, dK, dV, dQg, dKg, dVg};
  const int n_out = proj ? 6 : 3;
  for (int x = 0; x < n_out; ++x) {
    for (const void* in : {Q, K, V, O, dO, Qg, Kg, Vg})
      if (overlaps2(outs[x], out_b, in, in_b)) return LFATTN_EINVAL;
    if (overlaps2(outs[x], out_b, LSE, lse_b)) return LFATTN_EINVAL;
    for (int y = x + 1; y < n_out; ++y)
      if (overlaps2(outs[x], out_b, outs[y], out_b)) return LFATTN_EINVAL;
  }
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != c->device) return LFATTN_EINVAL;

  lfattn::BwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO; a.lse = LSE; a.terms = c->d_terms;
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.Qg = Qg; a.Kg = Kg; a.Vg = Vg;
  a.dQg = proj ? dQg : nullptr; a.dKg = proj ? dKg : nullptr; a.dVg = proj ? dVg : nullptr;
  a.proj = proj ? 1 : 0;
  a.glob = c->d_glob; a.is_glob = c->d_isglob;
  a.isg_stride = c->shared ? 0 : c->N;
  a.H = c->H; a.N = c->N; a.D = c->D; a.n_bh = c->B * c->H;
  a.hw = c->hw; a.hr = c->causal ? 0 : c->hw; a.chunk = c->chunk; a.cbase = c->n_memory;
  a.chunk_keys = c->bwd_chunk; a.n_glob = c->n_gmax;
  a.gpart = c->d_gpart; a.n_gch = c->n_gch; a.gsel = c->d_gsel;
  a.scale = c->scale; a.sl2 = c->scale * 1.4426950408889634f;
  a.rows_wpe = c->bwd_rows_wpe;
  // The key side: the same arguments with its own table and item size.
  lfattn::BwdArgs ak = a;
  a.work = c->d_bwork;
  a.ks = c->bwd_rows[0] == 64 ? 2 : 1;
  ak.work = c->d_bwork + c->n_bwork[0];
  ak.ks = c->bwd_rows[1] == 64 ? 2 : 1;
  lfattn::Timing t[3];
  const bool timed = c->timing && c->n_btimed < kMaxTimedBackwards;
  if (timed) {
    hipEvent_t* e = &c->bev[kEvPerBackward * c->n_btimed++];
    for (int x = 0; x < 3; ++x) t[x] = {e[2 * x], e[2 * x + 1]};
  }
  c->last = stream;
  c->used = true;
  if (lfattn::launch_backward_bf16(a, ak, c->n_bwork[0], c->n_bwork[1], stream, t) != hipSuccess)
    return LFATTN_EHIP;
  return LFATTN_OK;
}

}  // namespace

extern "C" {

lfattn_status lfattn_backward(lfattn_t c, const void* Q, const void* K, const void* V,
                              const void* O, const void* dO, const float* LSE, float* dQ,
                              float* dK, float* dV, hipStream_t stream) {
  return backward_impl(c, Q, K, V, nullptr, nullptr, nullptr, O, dO, LSE, dQ, dK, dV, nullptr,
                       nullptr, nullptr, false, stream);
}

lfattn_status lfattn_backward_global_proj(lfattn_t c, const void* Q, const void* K,
                                          const void* V, const void* Qg, const void* Kg,
                                          const void* Vg, const void* O, const void* dO,
                                          const float* LSE, float* dQ, float* dK, float* dV,
                                          float* dQg, float* dKg, float* dVg,
                                          hipStream_t stream) {
  return backward_impl(c, Q, K, V, Qg, Kg, Vg, O, dO, LSE, dQ, dK, dV, dQg, dKg, dVg, true,
                       stream);
}

lfattn_status lfattn_destroy(lfattn_t c) {
  if (!c) return LFATTN_OK;
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
  const long long glob_rows = (long long)c->H * c->n_gsum * c->N;
  *pairs = c->glob_items ? c->pairs : c->pairs - glob_rows;
  return LFATTN_OK;
}

lfattn_status lfattn_band_rows(lfattn_t c, int* rows) {
  if (!c || !rows) return LFATTN_EINVAL;
  *rows = c->band_rows;
  return LFATTN_OK;
}

lfattn_status lfattn_global_list(lfattn_t c, int* out, int capacity, int* n_out) {
  return lfattn_global_list_batch(c, 0, out, capacity, n_out);
}

lfattn_status lfattn_global_list_batch(lfattn_t c, int b, int* out, int capacity, int* n_out) {
  if (!c || !n_out || capacity < 0 || (capacity > 0 && !out)) return LFATTN_EINVAL;
  if (b < 0 || b >= c->B) return LFATTN_EINVAL;
  const std::vector<int>& g = c->G(b);
  const int n = (int)g.size();
  for (int t = 0; t < n && t < capacity; ++t) out[t] = g[t];
  *n_out = n;
  return LFATTN_OK;
}

lfattn_status lfattn_set_timing(lfattn_t c, int enable) {
  if (!c) return LFATTN_EINVAL;
  auto make = [](std::vector<hipEvent_t>& v, size_t n) {
    if (!v.empty()) return true;
    v.resize(n, nullptr);
    for (auto& e : v)
      if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        for (auto& x : v)
          if (x) (void)hipEventDestroy(x);
        v.clear();
        return false;
      }
    return true;
  };
  if (enable && (!make(c->ev, (size_t)kEvPerForward * kMaxTimedForwards) ||
                 !make(c->bev, (size_t)kEvPerBackward * kMaxTimedBackwards)))
    return LFATTN_EHIP;
  c->timing = enable != 0;
  c->n_timed = 0;
  c->n_btimed = 0;
  return LFATTN_OK;
}

lfattn_status lfattn_read_timing(lfattn_t c, double* band_ms, double* global_ms, int* n_forwards) {
  if (!c || !band_ms || !global_ms || !n_forwards) return LFATTN_EINVAL;
  double b = 0.0, g = 0.0;
  // Global-row kernels besides the band launch: the partials (fp32) and the
  // merge (unless the band launch merges).
  const bool has_glob = c->n_gmax > 0 && !c->fuse_merge;
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

lfattn_status lfattn_read_backward_timing(lfattn_t c, double* rows_ms, double* keys_ms,
                                          double* merge_ms, int* n_backwards) {
  if (!c || !rows_ms || !keys_ms || !merge_ms || !n_backwards) return LFATTN_EINVAL;
  double sum[3] = {0.0, 0.0, 0.0};
  // Kernels that a call does not launch record no events: none without work
  // items (an empty problem), the merge without global positions.
  const bool run = c->n_bwork[0] > 0 && c->n_bwork[1] > 0;
  const int n_k = !run ? 0 : (c->n_gmax > 0 ? 3 : 2);
  if (c->n_btimed > 0 && n_k > 0 &&
      hipEventSynchronize(c->bev[kEvPerBackward * (c->n_btimed - 1) + 2 * n_k - 1]) !=
          hipSuccess)
    return LFATTN_EHIP;
  for (int t = 0; t < c->n_btimed; ++t) {
    hipEvent_t* e = &c->bev[kEvPerBackward * t];
    for (int x = 0; x < n_k; ++x) {
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, e[2 * x], e[2 * x + 1]) != hipSuccess) return LFATTN_EHIP;
      sum[x] += ms;
    }
  }
  *rows_ms = sum[0];
  *keys_ms = sum[1];
  *merge_ms = sum[2];
  *n_backwards = c->n_btimed;
  c->n_btimed = 0;
  return LFATTN_OK;
}

}  // extern "C"
