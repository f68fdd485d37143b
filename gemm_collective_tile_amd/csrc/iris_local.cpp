// C-ABI host library: validation, configuration, workspace, launch and the
// gemm_wgs sweep for one GPU's share of the fused communication + GEMM ops.
//
// Operation definitions: Iris docs "Fused Communication and Compute
// Operations" (all_gather_matmul, matmul_reduce_scatter, matmul_all_reduce).
// Scheduling knobs, fused/sequential modes and the tuning policy (benchmark
// the candidates including the static default, keep the winner in a cache
// written to a temporary file then renamed, ignore a failed write, key by
// the device's gcnArchName): ROCm/iris PR "Add iris.concurrent (concurrent,
// independent, fused comm+gemm)", description and its autotune code excerpts.
// config == NULL selecting a configuration automatically and the NN-only
// layout: ROCm/iris PR "Add auto-config selection for fused AG+matmul with
// 28 tuned HBM buffer configs", summary.
#include "../../include/iris_local.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cerrno>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <sys/stat.h>
#include <unistd.h>
#include <vector>

#include "launch.hpp"
#include "mfma_ceiling.hpp"

namespace {

using iris::Params;

thread_local std::string g_msg;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_msg = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(IRIS_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// ------------------------------------------------------------ device facts
struct DevInfo {
  bool ok = false;
  int cus = 0;
  int clock_khz = 0, mem_clock_khz = 0, wall_khz = 0, lds = 0;
  int64_t mem = 0;
  std::string arch;
};

std::mutex g_mu;
std::map<int, DevInfo> g_dev;

int current_device(int* dev, DevInfo* info) {
  int d = 0;
  hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_dev.find(d);
    if (it != g_dev.end()) {
      *dev = d;
      *info = it->second;
      return IRIS_OK;
    }
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, d);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  DevInfo di;
  di.cus = prop.multiProcessorCount;
  di.clock_khz = prop.clockRate;
  di.mem_clock_khz = prop.memoryClockRate;
  di.lds = (int)prop.maxSharedMemoryPerMultiProcessor;
  di.mem = (int64_t)prop.totalGlobalMem;
  di.arch = prop.gcnArchName;
  int wall = 0;
  if (hipDeviceGetAttribute(&wall, hipDeviceAttributeWallClockRate, d) != hipSuccess) wall = 100000;
  di.wall_khz = wall > 0 ? wall : 100000;
  di.ok = di.arch.rfind("gfx950", 0) == 0;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_dev[d] = di;
  }
  *dev = d;
  *info = di;
  if (!di.ok) return fail(IRIS_ERR_NO_DEVICE, "device %d is %s; this library is built for gfx950", d, di.arch.c_str());
  return IRIS_OK;
}

// ------------------------------------------------------------ tuning cache
std::string cache_path() {
  const char* p = getenv("IRIS_LOCAL_TUNE_CACHE");
  if (p && *p) return p;
  const char* home = getenv("HOME");
  return std::string(home && *home ? home : "/tmp") + "/.cache/iris_local/tune.json";
}

std::string cache_key(const std::string& arch, int op, int64_t M, int64_t N, int64_t K, int W, int bm,
                      int bn, int bk, int gm) {
  char buf[256];
  std::string a = arch.substr(0, arch.find(':'));
  snprintf(buf, sizeof buf, "%s op%d M%lld N%lld K%lld W%d t%dx%dx%d g%d", a.c_str(), op, (long long)M,
           (long long)N, (long long)K, W, bm, bn, bk, gm);
  return buf;
}

// The cache is one JSON object mapping a key string to the tuned gemm_wgs,
// e.g. {"gfx950 op1 M4096 N4096 K512 W8 t256x256x64 g8": 1}. The reader
// accepts exactly that shape (string keys with \" and \\ escapes, integer
// values, any white space); a file it cannot parse is treated as empty.
struct JsonIn {
  const std::string& s;
  size_t i = 0;
  void ws() {
    while (i < s.size() && (s[i] == ' ' || s[i] == '\n' || s[i] == '\t' || s[i] == '\r')) ++i;
  }
  bool eat(char c) {
    ws();
    if (i < s.size() && s[i] == c) {
      ++i;
      return true;
    }
    return false;
  }
  bool str(std::string* out) {
    if (!eat('"')) return false;
    out->clear();
    while (i < s.size() && s[i] != '"') {
      char c = s[i++];
      if (c == '\\') {
        if (i >= s.size()) return false;
        c = s[i++];
        if (c != '"' && c != '\\' && c != '/') return false;
      }
      out->push_back(c);
    }
    return eat('"');
  }
  bool integer(long* out) {
    ws();
    const char* b = s.c_str() + i;
    char* e = nullptr;
    errno = 0;
    const long v = strtol(b, &e, 10);
    if (e == b || errno != 0) return false;
    i += (size_t)(e - b);
    *out = v;
    return true;
  }
};

std::map<std::string, int> parse_cache(const std::string& text) {
  std::map<std::string, int> db;
  JsonIn in{text};
  if (!in.eat('{')) return {};
  if (in.eat('}')) return db;
  do {
    std::string k;
    long v = 0;
    if (!in.str(&k) || !in.eat(':') || !in.integer(&v)) return {};
    if (v > 0 && v < (1 << 20)) db[k] = (int)v;
  } while (in.eat(','));
  if (!in.eat('}')) return {};
  return db;
}

std::map<std::string, int> load_cache() {
  FILE* f = fopen(cache_path().c_str(), "r");
  if (!f) return {};
  std::string text;
  char buf[4096];
  size_t n;
  while ((n = fread(buf, 1, sizeof buf, f)) > 0) text.append(buf, n);
  fclose(f);
  return parse_cache(text);
}

std::string json_escape(const std::string& k) {
  std::string o;
  for (char c : k) {
    if (c == '"' || c == '\\') o.push_back('\\');
    o.push_back(c);
  }
  return o;
}

void mkdirs(const std::string& path) {
  for (size_t i = 1; i < path.size(); ++i)
    if (path[i] == '/') mkdir(path.substr(0, i).c_str(), 0755);
}

void save_cache_entry(const std::string& key, int value) {
  std::map<std::string, int> db = load_cache();
  db[key] = value;
  const std::string path = cache_path();
  mkdirs(path);
  const std::string tmp = path + "." + std::to_string(getpid()) + ".tmp";
  FILE* f = fopen(tmp.c_str(), "w");
  if (!f) return;  // an unwritable cache only loses the memo
  bool ok = fputs("{\n", f) >= 0;
  size_t i = 0;
  for (auto& kv : db)
    ok = ok && fprintf(f, "  \"%s\": %d%s\n", json_escape(kv.first).c_str(), kv.second,
                       ++i < db.size() ? "," : "") > 0;
  ok = ok && fputs("}\n", f) >= 0;
  ok = (fclose(f) == 0) && ok;
  if (!ok || rename(tmp.c_str(), path.c_str()) != 0) unlink(tmp.c_str());
}

// The cache file is read once per path and process; later tunings in this
// process update the in-memory copy, so an op call costs no file access.
std::mutex g_cache_mu;
std::string g_cache_path;
std::map<std::string, int> g_cache;
bool g_cache_loaded = false;

int tuned_gemm_wgs(const std::string& key) {
  std::lock_guard<std::mutex> lk(g_cache_mu);
  const std::string path = cache_path();
  if (!g_cache_loaded || path != g_cache_path) {
    g_cache = load_cache();
    g_cache_path = path;
    g_cache_loaded = true;
  }
  auto it = g_cache.find(key);
  return it == g_cache.end() ? 0 : it->second;
}

void remember_gemm_wgs(const std::string& key, int value) {
  std::lock_guard<std::mutex> lk(g_cache_mu);
  save_cache_entry(key, value);
  const std::string path = cache_path();
  if (g_cache_loaded && path == g_cache_path) g_cache[key] = value;
}

// --------------------------------------------------------------- config
struct Resolved {
  int bm, bn, bk, gm, gemm_wgs, comm_bm, comm_bn, comm_chunk, mode, flags;
  int grid;
};

constexpr int kDefaultTile = 256;
constexpr int kDefaultGroupM = 8;
constexpr int kDefaultChunk = 65536;

int iris_op_to_kind(int op) {
  switch (op) {
    case IRIS_OP_AG_MM: return iris::OP_AG;
    case IRIS_OP_MM_RS: return iris::OP_RS;
    case IRIS_OP_MM_AR: return iris::OP_ARMM;
    case IRIS_OP_CONCURRENT: return iris::OP_CONC_AR;
    case IRIS_OP_MM_AG: return iris::OP_CONC_COPY;
  }
  return -1;
}

// Validates and fills everything but the grid / gemm_wgs (device-dependent).
int resolve_static(const iris_config_t* cfg, Resolved* r) {
  iris_config_t c{};
  if (cfg) c = *cfg;
  r->bm = c.block_m > 0 ? c.block_m : kDefaultTile;
  r->bn = c.block_n > 0 ? c.block_n : kDefaultTile;
  if (c.block_m <= 0 && c.block_n > 0) r->bm = c.block_n == 64 ? 64 : (c.block_n == 128 ? 128 : 256);
  if (c.block_n <= 0 && c.block_m > 0) r->bn = c.block_m == 64 ? 64 : (c.block_m == 128 ? 128 : 256);
  r->bk = c.block_k > 0 ? c.block_k : 64;
  r->gm = c.group_m > 0 ? c.group_m : kDefaultGroupM;
  r->gemm_wgs = c.gemm_wgs;
  r->comm_bm = c.comm_block_m > 0 ? c.comm_block_m : 0;  // 0: chosen per op in run()
  r->comm_bn = c.comm_block_n > 0 ? c.comm_block_n : r->bn;
  r->comm_chunk = c.comm_chunk > 0 ? c.comm_chunk : kDefaultChunk;
  r->mode = c.mode;
  r->flags = c.flags;
  if (!iris::tile_supported(r->bm, r->bn))
    return fail(IRIS_ERR_CONFIG, "unsupported GEMM tile %dx%d (supported: 256x256, 256x128, 128x128, 64x64)",
                r->bm, r->bn);
  if (r->bk != 64) return fail(IRIS_ERR_CONFIG, "block_k must be 64 (got %d)", r->bk);
  if (r->gm > 1 << 16) return fail(IRIS_ERR_CONFIG, "group_m too large (%d)", r->gm);
  if (r->comm_bm > 0 && r->bm % r->comm_bm != 0)
    return fail(IRIS_ERR_CONFIG, "comm_block_m must divide block_m (%d does not divide %d)", r->comm_bm, r->bm);
  if (r->comm_bn % 8 != 0) return fail(IRIS_ERR_CONFIG, "comm_block_n must be a multiple of 8 (got %d)", r->comm_bn);
  if (r->comm_chunk % 2048 != 0) return fail(IRIS_ERR_CONFIG, "comm_chunk must be a multiple of 2048 (got %d)", r->comm_chunk);
  if (r->mode != IRIS_MODE_FUSED && r->mode != IRIS_MODE_SEQUENTIAL && r->mode != IRIS_MODE_TWO_STREAM)
    return fail(IRIS_ERR_CONFIG, "unknown mode %d", r->mode);
  if (r->flags & ~(IRIS_FLAG_NO_STEAL | IRIS_FLAG_BIAS_ALONG_M | IRIS_FLAG_NO_LOCKSTEP))
    return fail(IRIS_ERR_CONFIG, "unknown flag bits 0x%x", r->flags);
  return IRIS_OK;
}

int resolve_device(Resolved* r, int kind, const DevInfo& di, const std::string& key) {
  const int occ = iris::persistent_blocks_per_cu(r->bm, r->bn, kind);
  if (occ <= 0) return fail(IRIS_ERR_HIP, "occupancy query failed for tile %dx%d", r->bm, r->bn);
  r->grid = di.cus * occ;
  if (r->grid > 2048) r->grid = 2048;
  if (r->gemm_wgs <= 0) {
    const int tuned = r->mode == IRIS_MODE_FUSED ? tuned_gemm_wgs(key) : 0;
    r->gemm_wgs = (tuned > 0 && tuned < r->grid) ? tuned : (r->grid * 7) / 8;
  }
  if (r->mode != IRIS_MODE_SEQUENTIAL && (r->gemm_wgs < 1 || r->gemm_wgs > r->grid - 1))
    return fail(IRIS_ERR_CONFIG, "gemm_wgs %d outside [1, %d] for a grid of %d workgroups", r->gemm_wgs,
                r->grid - 1, r->grid);
  return IRIS_OK;
}

// Rows per comm unit when the config leaves it open: the largest power of
// two dividing block_m that keeps a unit near a target size, 128 KiB of
// shard for a copy unit and 32 KiB per buffer for a reduce unit. Units that
// small let many workgroups share one GEMM row block, so the first blocks
// are ready early, while each unit stays far above the cost of its claim
// and release.
int default_comm_rows(int kind, int bm, int64_t row_bytes) {
  const int64_t target = kind == iris::OP_AG ? 131072 : 32768;
  int rows = bm;
  while (rows > 1 && (int64_t)rows * row_bytes > target) rows >>= 1;
  return rows;
}

// ------------------------------------------------------------- workspace
constexpr int kMaxGrid = iris::kMaxGrid;
constexpr size_t kStampBytes = (size_t)kMaxGrid * iris::kStampWords * sizeof(uint64_t);

int64_t flag_words(int kind, int64_t M, int64_t N, int W, int bm, int bn) {
  const int64_t n_pm = (M + bm - 1) / bm, n_pn = (N + bn - 1) / bn;
  if (kind == iris::OP_AG) return n_pm * iris::kLine;
  if (kind == iris::OP_RS || kind == iris::OP_ARMM) return n_pm * n_pn;
  return 0;
}

size_t int_region_bytes(int64_t words) {
  const size_t b = (size_t)(iris::kFlagBase + words) * 4;
  return (b + 255) & ~(size_t)255;
}

struct OwnedWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::map<std::pair<int, void*>, OwnedWs> g_ws;   // (device, stream) -> workspace
struct LastLaunch {
  int dev;
  int grid;          // workgroups of the persistent launch
  int comm_grid;     // workgroups of the sequential comm kernel (0 if fused)
  bool fused;
  size_t stamp_off;  // byte offset of the stamps in the workspace (0)
};
std::map<void*, LastLaunch> g_last;  // workspace -> its last launch

int get_workspace(int dev, void* stream, size_t need, void* user, size_t user_bytes, void** out) {
  if (user) {
    if (user_bytes < need)
      return fail(IRIS_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", user_bytes, need);
    if ((uintptr_t)user % 256 != 0) return fail(IRIS_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
    *out = user;
    return IRIS_OK;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  OwnedWs& w = g_ws[{dev, stream}];
  if (w.bytes < need) {
    if (w.ptr) {
      // the old buffer may still be in use by enqueued work on this stream
      hipError_t e = hipStreamSynchronize((hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    size_t bytes = std::max(need, (size_t)1 << 20);
    hipError_t e = hipMalloc(&w.ptr, bytes);
    if (e != hipSuccess) {
      w.ptr = nullptr;
      return fail(IRIS_ERR_NO_MEMORY, "hipMalloc of a %zu-byte workspace failed: %s", bytes, hipGetErrorString(e));
    }
    // a fresh workspace starts zeroed; every op leaves it zeroed again
    e = hipMemsetAsync(w.ptr, 0, bytes, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "workspace clear");
    w.bytes = bytes;
  }
  *out = w.ptr;
  return IRIS_OK;
}

// ------------------------------------------------------------ validation
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int check_ptr(const void* p, const char* name, bool required = true) {
  if (!p) return required ? fail(IRIS_ERR_INVALID_ARG, "%s is NULL", name) : IRIS_OK;
  if (!aligned16(p)) return fail(IRIS_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  return IRIS_OK;
}

int check_gemm_dims(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(IRIS_ERR_INVALID_ARG, "M, N, K must be positive (got %lld, %lld, %lld)",
                                               (long long)M, (long long)N, (long long)K);
  if (M > (1 << 30) || N > (1 << 21) || K > (1 << 21))
    return fail(IRIS_ERR_UNSUPPORTED, "shape too large (limits: M <= 2^30, N <= 2^21, K <= 2^21)");
  if (N % 8 != 0 || K % 8 != 0)
    return fail(IRIS_ERR_ALIGNMENT, "N and K must be multiples of 8 (got N=%lld, K=%lld)", (long long)N, (long long)K);
  return IRIS_OK;
}

// ---------------------------------------------------------------- launch
struct OpDesc {
  int kind;        // iris::OpKind
  int iris_op;     // IRIS_OP_* (tuning cache key)
  int collective;  // IRIS_COLL_* of the concurrent op, else 0
  void* C;
  void* out;
  const void* A;
  const void* const* srcs;
  int W;      // ranks (AG: shards; RS/AR: ranks incl. own; concurrent: buffers)
  int rank;
  const void* B;
  const void* bias;
  int64_t M, N, K;  // K = full contraction length
  int64_t K_local;
  int64_t comm_elems;
  // flat comm units of the independent ops: sources W (reduce) or nsrc (copy)
  int64_t src_off;      // element offset applied to every source
  int64_t flat_elems;   // reduce: elements of the result; copy: block length
  int nsrc;             // copy: number of source blocks
  int dst_blk[IRIS_MAX_W];
};

// The second stream and fork/join events of the two-stream mode, per
// (device, caller stream), created on first use.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::map<std::pair<int, void*>, SideStream> g_side;

int get_side_stream(int dev, void* stream, SideStream** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  SideStream& ss = g_side[{dev, stream}];
  if (!ss.s) {
    hipError_t e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (ss.join) (void)hipEventDestroy(ss.join);
      if (ss.fork) (void)hipEventDestroy(ss.fork);
      if (ss.s) (void)hipStreamDestroy(ss.s);
      ss = SideStream{};
      return hip_fail(e, "creating the two-stream mode's stream and events");
    }
  }
  *out = &ss;
  return IRIS_OK;
}

// Waits for `stream`, then reads and clears the status word of workspace
// `ws`: the timeout bit is set by the last workgroup of any fused launch in
// which a device-side wait gave up, and stays set until read here.
int read_status(void* ws, hipStream_t s) {
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int32_t* word = (int32_t*)((char*)ws + kStampBytes) + iris::kStatus;
  int32_t v = 0;
  e = hipMemcpy(&v, word, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "status readback");
  if (v == 0) return IRIS_OK;
  e = hipMemset(word, 0, 4);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "status clear");
  return fail(IRIS_ERR_DEVICE_TIMEOUT, "a device-side wait hit its poll bound; the outputs of the ops since the "
              "last check are not to be trusted");
}

int run(const OpDesc& d, const iris_config_t* cfg, void* workspace, size_t ws_bytes, void* stream,
        Resolved* used = nullptr) {
  Resolved r{};
  int st = resolve_static(cfg, &r);
  if (st) return st;
  if (r.mode == IRIS_MODE_TWO_STREAM && d.kind != iris::OP_CONC_AR && d.kind != iris::OP_CONC_COPY)
    return fail(IRIS_ERR_CONFIG,
                "two-stream mode needs an op whose GEMM and collective are independent "
                "(iris_concurrent, iris_mm_ag_local)");
  // the tile count depends on the shape and the tile only: checked before
  // any device call, like every other argument
  if (((d.M + r.bm - 1) / r.bm) * ((d.N + r.bn - 1) / r.bn) > (1 << 30))
    return fail(IRIS_ERR_UNSUPPORTED, "too many GEMM tiles (%lld; limit 2^30)",
                (long long)(((d.M + r.bm - 1) / r.bm) * ((d.N + r.bn - 1) / r.bn)));
  int dev = 0;
  DevInfo di;
  st = current_device(&dev, &di);
  if (st) return st;
  // the concurrent op's collectives tune apart: fold the collective into the op
  const std::string key = cache_key(di.arch, d.iris_op * 16 + d.collective, d.M, d.N,
                                    d.kind == iris::OP_AG ? d.K_local : d.K, d.W, r.bm, r.bn, r.bk, r.gm);
  st = resolve_device(&r, d.kind, di, key);
  if (st) return st;
  if (r.comm_bm <= 0) {
    const int64_t row_bytes = d.kind == iris::OP_AG ? d.K_local * 2
                              : d.kind == iris::OP_CONC_AR
                                  ? 0
                                  : std::min<int64_t>(r.comm_bn, d.kind == iris::OP_RS ? d.N / d.W : d.N) * 2;
    r.comm_bm = default_comm_rows(d.kind, r.bm, row_bytes);
    while (d.kind == iris::OP_AG && r.comm_bm > 1 && (int64_t)r.comm_bm * d.K * 2 >= (int64_t)1 << 31)
      r.comm_bm >>= 1;
  }
  // a copy unit addresses its gathered rows through one 32-bit buffer range
  if (d.kind == iris::OP_AG && (int64_t)r.comm_bm * d.K * 2 >= (int64_t)1 << 31)
    return fail(IRIS_ERR_CONFIG, "comm_block_m %d times the gathered row (%lld bytes) exceeds 2 GiB", r.comm_bm,
                (long long)(d.K * 2));
  if (used) *used = r;

  const int64_t words = flag_words(d.kind, d.M, d.N, d.W, r.bm, r.bn);
  const size_t ibytes = int_region_bytes(words);
  void* ws = nullptr;
  st = get_workspace(dev, stream, ibytes + kStampBytes, workspace, ws_bytes, &ws);
  if (st) return st;

  Params p;
  memset(&p, 0, sizeof p);
  iris::GemmArgs& g = p.g;
  g.A = (const iris::f16*)(d.kind == iris::OP_AG ? d.out : d.A);
  g.lda = d.K;
  g.B = (const iris::f16*)d.B;
  g.ldb = d.N;
  g.bias = (const iris::f16*)d.bias;
  g.bias_along_m = (r.flags & IRIS_FLAG_BIAS_ALONG_M) ? 1 : 0;
  g.C = (iris::f16*)d.C;
  g.ldc = d.N;
  g.M = (int)d.M;
  g.N = (int)d.N;
  g.K = (int)d.K;
  const int n_pm = (int)((d.M + r.bm - 1) / r.bm);
  const int n_pn = (int)((d.N + r.bn - 1) / r.bn);
  p.order.n_pm = n_pm;
  p.order.n_pn = n_pn;
  p.order.group_m = r.gm;
  p.T_gemm = n_pm * n_pn;
  p.xcd_q = std::max(1, r.grid / iris::kXcds);
  iris::CommArgs& c = p.c;
  int64_t t_comm = 0;
  c.M = (int)d.M;
  c.BM = r.bm;
  c.rows_u = r.comm_bm;
  c.n_sub = r.bm / r.comm_bm;
  switch (d.kind) {
    case iris::OP_AG:
      c.W = d.W;
      for (int s = 0; s < d.W; ++s) c.src[s] = (const iris::f16*)d.srcs[s];
      c.dst = (iris::f16*)d.out;
      c.K_local = d.K_local;
      c.K = d.K;
      t_comm = (int64_t)n_pm * d.W * c.n_sub;
      break;
    case iris::OP_RS:
    case iris::OP_ARMM: {
      const int64_t nl = d.kind == iris::OP_RS ? d.N / d.W : d.N;
      c.W = d.W - 1;
      for (int s = 0; s < d.W - 1; ++s) c.src[s] = (const iris::f16*)d.srcs[s];
      c.dst = (iris::f16*)d.out;
      c.C = (const iris::f16*)d.C;
      c.ldc = d.N;
      c.col0 = d.kind == iris::OP_RS ? (int)(d.rank * nl) : 0;
      c.ncols = (int)nl;
      c.comm_bn = r.comm_bn;
      c.n_cc = (int)((nl + r.comm_bn - 1) / r.comm_bn);
      t_comm = (int64_t)n_pm * c.n_sub * c.n_cc;
      // GEMM tiles feeding this rank's slice go first
      p.order.prio_lo = c.col0 / r.bn;
      p.order.prio_hi = (int)((c.col0 + nl + r.bn - 1) / r.bn);
      break;
    }
    case iris::OP_CONC_AR:
      c.W = d.W;
      for (int s = 0; s < d.W; ++s) c.src[s] = (const iris::f16*)d.srcs[s] + d.src_off;
      c.dst = (iris::f16*)d.out;
      c.elems = d.flat_elems;
      c.chunk = r.comm_chunk;
      t_comm = (d.flat_elems + r.comm_chunk - 1) / r.comm_chunk;
      break;
    case iris::OP_CONC_COPY:
      c.W = d.nsrc;
      for (int s = 0; s < d.nsrc; ++s) {
        c.src[s] = (const iris::f16*)d.srcs[s] + d.src_off;
        c.dst_blk[s] = d.dst_blk[s];
      }
      c.dst = (iris::f16*)d.out;
      c.blk = d.flat_elems;
      c.chunk = r.comm_chunk;
      c.n_chunk = (int)((d.flat_elems + r.comm_chunk - 1) / r.comm_chunk);
      t_comm = (int64_t)d.nsrc * c.n_chunk;
      break;
  }
  if (t_comm > (1 << 30))
    return fail(IRIS_ERR_UNSUPPORTED, "too many comm units (%lld; limit 2^30)", (long long)t_comm);
  p.T_comm = (int)t_comm;
  // Layout: the timestamp block at a fixed offset 0, then the counters and
  // flags. The flag region's size depends on the op; with the stamps first,
  // no op's stamps can land on another op's flag words.
  p.stamps = (uint64_t*)ws;
  p.ws = (int32_t*)((char*)ws + kStampBytes);
  p.comm_stamps = p.stamps + (size_t)kMaxGrid * 4;
  p.spin_limit = 1u << 24;
  if (const char* sl = getenv("IRIS_LOCAL_SPIN_LIMIT")) {
    char* end = nullptr;
    const long v = strtol(sl, &end, 10);
    if (end != sl && v >= 0 && v <= (1L << 30)) p.spin_limit = (uint32_t)v;
  }
  p.n_reset = (int)(ibytes / 4);
  p.steal = (r.flags & IRIS_FLAG_NO_STEAL) ? 0 : 1;
  const hipStream_t s = (hipStream_t)stream;

  hipError_t e = hipSuccess;
  int comm_grid = 0;
  int gemm_grid = r.grid;
  if (r.mode == IRIS_MODE_FUSED) {
    p.op = d.kind;
    p.fused = 1;
    p.gemm_wgs = r.gemm_wgs;
    // beside an independent collective only the gemm_wgs workgroups that
    // start on the GEMM run tiles for most of the launch: deal the XCD queues
    // in blocks of their number per XCD, so that the tiles an XCD runs at once
    // form whole patches (the concurrent 8192^3 GEMM at gemm_wgs 224:
    // 0.5-1.5 % faster on MI355X); the dependent ops run the GEMM on every
    // workgroup and keep blocks of grid / 8
    if (d.kind == iris::OP_CONC_AR || d.kind == iris::OP_CONC_COPY) p.xcd_q = std::max(1, r.gemm_wgs / iris::kXcds);
    // lockstep rounds only where an XCD queue is dealt in blocks of the
    // workgroups that work it: beside an independent collective more
    // workgroups join the GEMM than the blocks were sized for
    p.lockstep = p.xcd_q * iris::kXcds == r.grid && !(r.flags & IRIS_FLAG_NO_LOCKSTEP);
    e = iris::launch_persistent(p, r.bm, r.bn, r.grid, s);
    if (e != hipSuccess) return hip_fail(e, "fused launch");
  } else if (r.mode == IRIS_MODE_TWO_STREAM) {
    // fork: the comm kernel runs on the side stream after everything already
    // queued on the caller's stream; join: the caller's stream continues only
    // after it. The GEMM kernel takes gemm_wgs workgroups, the comm kernel
    // the rest of the CUs; neither waits on the other.
    SideStream* ss = nullptr;
    st = get_side_stream(dev, stream, &ss);
    if (st) return st;
    Params pg = p;
    pg.op = iris::OP_GEMM;
    pg.fused = 0;
    pg.T_comm = 0;
    pg.gemm_wgs = r.gemm_wgs;
    pg.xcd_q = std::max(1, r.gemm_wgs / iris::kXcds);
    pg.lockstep = pg.xcd_q * iris::kXcds == r.gemm_wgs && !(r.flags & IRIS_FLAG_NO_LOCKSTEP);
    Params pc = p;
    pc.op = d.kind;
    pc.fused = 0;
    gemm_grid = r.gemm_wgs;
    comm_grid = std::min((r.grid - r.gemm_wgs) * 4, kMaxGrid);
    e = hipEventRecord(ss->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->s, ss->fork, 0);
    if (e == hipSuccess) e = iris::launch_comm_only(pc, comm_grid, ss->s);
    if (e == hipSuccess) e = iris::launch_persistent(pg, r.bm, r.bn, gemm_grid, s);
    if (e == hipSuccess) e = hipEventRecord(ss->join, ss->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, ss->join, 0);
    if (e != hipSuccess) return hip_fail(e, "two-stream launch");
  } else {
    // unfused baseline: the comm kernel and the GEMM kernel each get the
    // whole GPU, in dependency order (gather before GEMM; GEMM before reduce)
    Params pg = p;
    pg.op = iris::OP_GEMM;
    pg.fused = 0;
    pg.T_comm = 0;
    pg.gemm_wgs = r.grid;
    pg.lockstep = pg.xcd_q * iris::kXcds == r.grid && !(r.flags & IRIS_FLAG_NO_LOCKSTEP);
    Params pc = p;
    pc.op = d.kind;
    pc.fused = 0;
    // A gather larger than the 256 MiB last-level cache runs on the
    // persistent kernel's body with no GEMM tiles: its copy workgroups, one per CU,
    // claim units one ahead from the shared queue (the g2 gather of 4 GiB:
    // 6.1 TB/s warm and 5.9 cold on MI355X, against 5.5 for the comm-only
    // kernel's fixed grid-strided units on 256 or 1024 workgroups). A smaller
    // gather, and the reduces, start sooner on the comm-only kernel's four
    // workgroups per CU (pow2_4k's 64 MiB: 3.6 TB/s cold against 3.4; the
    // 8 x 64Mi all_reduce: 5.6 against 5.35).
    const bool big_gather = d.kind == iris::OP_AG && (double)pc.c.M * (double)pc.c.K * 2.0 > 256.0 * (1 << 20);
    comm_grid = big_gather ? r.grid : std::min(di.cus * 4, kMaxGrid);
    if (d.kind == iris::OP_AG) {
      if (big_gather) {
        Params pq = pc;
        pq.T_gemm = 0;
        pq.gemm_wgs = 0;
        pq.lockstep = 0;
        e = iris::launch_gather_only(pq, r.bm, r.bn, r.grid, s);
      } else {
        e = iris::launch_comm_only(pc, comm_grid, s);
      }
      if (e == hipSuccess) e = iris::launch_persistent(pg, r.bm, r.bn, r.grid, s);
    } else {
      e = iris::launch_persistent(pg, r.bm, r.bn, r.grid, s);
      if (e == hipSuccess) e = iris::launch_comm_only(pc, comm_grid, s);
    }
    if (e != hipSuccess) return hip_fail(e, "sequential launch");
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_last[ws] = LastLaunch{dev, gemm_grid, comm_grid, r.mode == IRIS_MODE_FUSED, 0};
  }
  if (getenv("IRIS_LOCAL_DEBUG")) return read_status(ws, s);
  return IRIS_OK;
}

int copy_ptrs(const void* const* arr, int n, const char* name) {
  if (n > 0 && !arr) return fail(IRIS_ERR_INVALID_ARG, "%s array is NULL", name);
  for (int i = 0; i < n; ++i) {
    char nm[64];
    snprintf(nm, sizeof nm, "%s[%d]", name, i);
    int st = check_ptr(arr[i], nm);
    if (st) return st;
  }
  return IRIS_OK;
}

}  // namespace

// ====================================================================== ABI
namespace iris {
// Records the message for iris_last_error_message from the library's other
// translation units; returns status.
int set_error(int status, const char* msg) {
  g_msg = msg;
  return status;
}
}  // namespace iris

namespace {
// Arguments of iris_ag_mm and iris_ag_mm_noalloc, checked before any HIP call.
int check_ag_mm(void* C, void* A_gathered, const void* const* A_shards, int32_t W, const void* B,
                const void* bias, int64_t M, int64_t N, int64_t K_local) {
  if (W < 1 || W > IRIS_MAX_W) return fail(IRIS_ERR_INVALID_ARG, "W must be in [1, %d] (got %d)", IRIS_MAX_W, W);
  int st;
  if ((st = check_ptr(C, "C")) || (st = check_ptr(A_gathered, "A_gathered")) || (st = check_ptr(B, "B")) ||
      (st = check_ptr(bias, "bias", false)) || (st = copy_ptrs(A_shards, W, "A_shards")))
    return st;
  if (K_local <= 0) return fail(IRIS_ERR_INVALID_ARG, "K_local must be positive");
  if (K_local % 8 != 0) return fail(IRIS_ERR_ALIGNMENT, "K_local must be a multiple of 8 (got %lld)", (long long)K_local);
  return check_gemm_dims(M, N, K_local * W);
}
}  // namespace

extern "C" {

int iris_ag_mm(void* C, void* A_gathered, const void* const* A_shards, int32_t W, const void* B,
               const void* bias, int64_t M, int64_t N, int64_t K_local, const iris_config_t* cfg,
               void* workspace, size_t workspace_bytes, void* stream) {
  g_msg.clear();
  int st = check_ag_mm(C, A_gathered, A_shards, W, B, bias, M, N, K_local);
  if (st) return st;
  OpDesc d{};
  d.kind = iris::OP_AG;
  d.iris_op = IRIS_OP_AG_MM;
  d.C = C;
  d.out = A_gathered;
  d.srcs = A_shards;
  d.W = W;
  d.B = B;
  d.bias = bias;
  d.M = M;
  d.N = N;
  d.K = K_local * W;
  d.K_local = K_local;
  return run(d, cfg, workspace, workspace_bytes, stream);
}

int iris_ag_mm_noalloc(void* C, void* A_gathered, const void* const* A_shards, int32_t W, const void* B,
                       const void* bias, int64_t M, int64_t N, int64_t K_local, const iris_config_t* cfg,
                       void* stream) {
  g_msg.clear();
  int st = check_ag_mm(C, A_gathered, A_shards, W, B, bias, M, N, K_local);
  if (st) return st;
  Resolved r{};
  if ((st = resolve_static(cfg, &r))) return st;
  // the workspace this op needs is known from the shape and tile alone
  const size_t need = int_region_bytes(flag_words(iris::OP_AG, M, N, W, r.bm, r.bn)) + kStampBytes;
  if (need > iris::kScratchBytes)
    return fail(IRIS_ERR_WORKSPACE,
                "iris_ag_mm_noalloc needs %zu bytes of workspace for M=%lld with %dx%d tiles; its static scratch "
                "holds %zu (use iris_ag_mm with a workspace)",
                need, (long long)M, r.bm, r.bn, iris::kScratchBytes);
  int dev = 0;
  DevInfo di;
  if ((st = current_device(&dev, &di))) return st;
  void* ws = nullptr;
  const hipError_t e = iris::scratch_setup(dev, (hipStream_t)stream, &ws);
  if (e != hipSuccess) return hip_fail(e, "static scratch set-up");
  return iris_ag_mm(C, A_gathered, A_shards, W, B, bias, M, N, K_local, cfg, ws, iris::kScratchBytes, stream);
}

int iris_mm_rs_local(void* out, void* C, const void* A, const void* B, const void* bias,
                     const void* const* partials, int32_t W, int32_t rank, int64_t M, int64_t N, int64_t K,
                     const iris_config_t* cfg, void* workspace, size_t workspace_bytes, void* stream) {
  g_msg.clear();
  if (W < 1 || W > IRIS_MAX_W) return fail(IRIS_ERR_INVALID_ARG, "W must be in [1, %d] (got %d)", IRIS_MAX_W, W);
  if (rank < 0 || rank >= W) return fail(IRIS_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, W);
  int st;
  if ((st = check_ptr(out, "out")) || (st = check_ptr(C, "C")) || (st = check_ptr(A, "A")) ||
      (st = check_ptr(B, "B")) || (st = check_ptr(bias, "bias", false)) || (st = copy_ptrs(partials, W - 1, "partials")))
    return st;
  if ((st = check_gemm_dims(M, N, K))) return st;
  if (N % W != 0) return fail(IRIS_ERR_INVALID_ARG, "N (%lld) must be divisible by W (%d)", (long long)N, W);
  if ((N / W) % 8 != 0) return fail(IRIS_ERR_ALIGNMENT, "N/W must be a multiple of 8 (got %lld)", (long long)(N / W));
  OpDesc d{};
  d.kind = iris::OP_RS;
  d.iris_op = IRIS_OP_MM_RS;
  d.C = C;
  d.out = out;
  d.A = A;
  d.srcs = partials;
  d.W = W;
  d.rank = rank;
  d.B = B;
  d.bias = bias;
  d.M = M;
  d.N = N;
  d.K = K;
  return run(d, cfg, workspace, workspace_bytes, stream);
}

int iris_mm_ar_local(void* out, void* C, const void* A, const void* B, const void* bias,
                     const void* const* partials, int32_t W, int64_t M, int64_t N, int64_t K,
                     const iris_config_t* cfg, void* workspace, size_t workspace_bytes, void* stream) {
  g_msg.clear();
  if (W < 1 || W > IRIS_MAX_W) return fail(IRIS_ERR_INVALID_ARG, "W must be in [1, %d] (got %d)", IRIS_MAX_W, W);
  int st;
  if ((st = check_ptr(out, "out")) || (st = check_ptr(C, "C")) || (st = check_ptr(A, "A")) ||
      (st = check_ptr(B, "B")) || (st = check_ptr(bias, "bias", false)) || (st = copy_ptrs(partials, W - 1, "partials")))
    return st;
  if ((st = check_gemm_dims(M, N, K))) return st;
  OpDesc d{};
  d.kind = iris::OP_ARMM;
  d.iris_op = IRIS_OP_MM_AR;
  d.C = C;
  d.out = out;
  d.A = A;
  d.srcs = partials;
  d.W = W;
  d.B = B;
  d.bias = bias;
  d.M = M;
  d.N = N;
  d.K = K;
  return run(d, cfg, workspace, workspace_bytes, stream);
}

int iris_concurrent(void* C, const void* A, const void* B, const void* bias, int64_t M, int64_t N, int64_t K,
                    int32_t collective, int32_t rank, void* comm_out, const void* const* comm_in, int32_t W,
                    int64_t comm_elems, const iris_config_t* cfg, void* workspace, size_t workspace_bytes,
                    void* stream) {
  g_msg.clear();
  if (collective < IRIS_COLL_ALL_REDUCE || collective > IRIS_COLL_BROADCAST)
    return fail(IRIS_ERR_UNSUPPORTED, "unknown collective %d", collective);
  if (W < 1 || W > IRIS_MAX_W) return fail(IRIS_ERR_INVALID_ARG, "W must be in [1, %d] (got %d)", IRIS_MAX_W, W);
  const bool ranked = collective == IRIS_COLL_REDUCE_SCATTER || collective == IRIS_COLL_ALL_TO_ALL ||
                      collective == IRIS_COLL_BROADCAST;
  if (ranked && (rank < 0 || rank >= W)) return fail(IRIS_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, W);
  int st;
  if ((st = check_ptr(C, "C")) || (st = check_ptr(A, "A")) || (st = check_ptr(B, "B")) ||
      (st = check_ptr(bias, "bias", false)) || (st = check_ptr(comm_out, "comm_out")) ||
      (st = copy_ptrs(comm_in, W, "comm_in")))
    return st;
  if ((st = check_gemm_dims(M, N, K))) return st;
  const int64_t n = comm_elems;
  if (n <= 0) return fail(IRIS_ERR_INVALID_ARG, "comm_elems must be positive");
  if (n % 8 != 0) return fail(IRIS_ERR_ALIGNMENT, "comm_elems must be a multiple of 8");
  if (n > ((int64_t)1 << 40)) return fail(IRIS_ERR_UNSUPPORTED, "comm_elems too large");
  const bool split = collective == IRIS_COLL_REDUCE_SCATTER || collective == IRIS_COLL_ALL_TO_ALL;
  if (split && n % (8 * (int64_t)W) != 0)
    return fail(IRIS_ERR_ALIGNMENT, "comm_elems must be a multiple of 8 W for this collective (got %lld, W=%d)",
                (long long)n, W);
  OpDesc d{};
  d.iris_op = IRIS_OP_CONCURRENT;
  d.collective = collective;
  d.C = C;
  d.out = comm_out;
  d.A = A;
  d.srcs = comm_in;
  d.W = W;
  d.rank = rank;
  d.B = B;
  d.bias = bias;
  d.M = M;
  d.N = N;
  d.K = K;
  d.comm_elems = n;
  switch (collective) {
    case IRIS_COLL_ALL_REDUCE:  // every element, every buffer
      d.kind = iris::OP_CONC_AR;
      d.flat_elems = n;
      break;
    case IRIS_COLL_REDUCE_SCATTER:  // this rank's n/W slice of every buffer
      d.kind = iris::OP_CONC_AR;
      d.src_off = (int64_t)rank * (n / W);
      d.flat_elems = n / W;
      break;
    case IRIS_COLL_ALL_GATHER:  // buffer w -> block w of W n
      d.kind = iris::OP_CONC_COPY;
      d.nsrc = W;
      d.flat_elems = n;
      for (int w = 0; w < W; ++w) d.dst_blk[w] = w;
      break;
    case IRIS_COLL_ALL_TO_ALL:  // block `rank` of buffer j -> block j
      d.kind = iris::OP_CONC_COPY;
      d.nsrc = W;
      d.src_off = (int64_t)rank * (n / W);
      d.flat_elems = n / W;
      for (int w = 0; w < W; ++w) d.dst_blk[w] = w;
      break;
    case IRIS_COLL_BROADCAST:  // the root's buffer
      d.kind = iris::OP_CONC_COPY;
      d.nsrc = 1;
      d.srcs = comm_in + rank;
      d.flat_elems = n;
      d.dst_blk[0] = 0;
      break;
  }
  return run(d, cfg, workspace, workspace_bytes, stream);
}

int iris_mm_ag_local(void* out, const void* A, const void* B, const void* bias, const void* const* peer_blocks,
                     int32_t W, int32_t rank, int64_t M, int64_t N, int64_t K, const iris_config_t* cfg,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_msg.clear();
  if (W < 1 || W > IRIS_MAX_W) return fail(IRIS_ERR_INVALID_ARG, "W must be in [1, %d] (got %d)", IRIS_MAX_W, W);
  if (rank < 0 || rank >= W) return fail(IRIS_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, W);
  int st;
  if ((st = check_ptr(out, "out")) || (st = check_ptr(A, "A")) || (st = check_ptr(B, "B")) ||
      (st = check_ptr(bias, "bias", false)) || (st = copy_ptrs(peer_blocks, W - 1, "peer_blocks")))
    return st;
  if ((st = check_gemm_dims(M, N, K))) return st;
  if ((int64_t)W * M > (1 << 30)) return fail(IRIS_ERR_UNSUPPORTED, "M * W too large (limit 2^30)");
  OpDesc d{};
  d.kind = iris::OP_CONC_COPY;
  d.iris_op = IRIS_OP_MM_AG;
  // this rank's block of the output is the GEMM's C
  d.C = (char*)out + (size_t)rank * (size_t)M * (size_t)N * 2;
  d.out = out;
  d.A = A;
  d.srcs = peer_blocks;
  d.W = W;
  d.rank = rank;
  d.B = B;
  d.bias = bias;
  d.M = M;
  d.N = N;
  d.K = K;
  d.nsrc = W - 1;
  d.flat_elems = M * N;
  for (int p = 0; p < W - 1; ++p) d.dst_blk[p] = p < rank ? p : p + 1;
  return run(d, cfg, workspace, workspace_bytes, stream);
}

size_t iris_workspace_size(int32_t op, int64_t M, int64_t N, int64_t K, int32_t W, const iris_config_t* cfg) {
  (void)K;
  Resolved r{};
  if (resolve_static(cfg, &r)) return 0;
  const int kind = iris_op_to_kind(op);
  if (kind < 0 || M <= 0 || N <= 0 || W < 1 || W > IRIS_MAX_W) return 0;
  return int_region_bytes(flag_words(kind, M, N, W, r.bm, r.bn)) + kStampBytes;
}

int iris_grid_size(int32_t op, const iris_config_t* cfg) {
  g_msg.clear();
  const int kind = iris_op_to_kind(op);
  if (kind < 0) return -fail(IRIS_ERR_INVALID_ARG, "unknown op %d", op);
  Resolved r{};
  int st = resolve_static(cfg, &r);
  if (st) return -st;
  int dev;
  DevInfo di;
  st = current_device(&dev, &di);
  if (st) return -st;
  const int occ = iris::persistent_blocks_per_cu(r.bm, r.bn, kind);
  if (occ <= 0) return -fail(IRIS_ERR_HIP, "occupancy query failed");
  return std::min(di.cus * occ, kMaxGrid);
}

int iris_tune_gemm_wgs(const iris_op_args_t* a, const int32_t* candidates, int32_t n_candidates, int32_t reps,
                       int32_t top_k, int32_t* best_gemm_wgs, float* ms_out, void* stream) {
  g_msg.clear();
  if (!a || !best_gemm_wgs) return fail(IRIS_ERR_INVALID_ARG, "args and best_gemm_wgs must not be NULL");
  if (n_candidates < 0 || (n_candidates > 0 && !candidates))
    return fail(IRIS_ERR_INVALID_ARG, "bad candidate list");
  if (reps < 1) reps = 5;
  iris_config_t cfg = a->cfg;
  cfg.mode = IRIS_MODE_FUSED;
  // the static default is always benchmarked, so tuning never loses to it
  int G = iris_grid_size(a->op, &cfg);
  if (G < 0) return -G;
  std::vector<int> cands(candidates, candidates + n_candidates);
  std::vector<int> bench_idx;  // position in `candidates` of each benchmarked candidate
  for (int i = 0; i < n_candidates; ++i) bench_idx.push_back(i);
  if (top_k > 0 && top_k < n_candidates) {
    std::vector<float> pred((size_t)n_candidates);
    const int ps = iris_predict_gemm_wgs(a, G, candidates, n_candidates, nullptr, pred.data(), nullptr);
    if (ps) return fail(ps, "the split predictor rejected the op or a candidate");
    const auto mm = std::minmax_element(pred.begin(), pred.end());
    // a flat prediction cannot rank: then every candidate is benchmarked
    if (*mm.second - *mm.first > 1e-6f * *mm.second) {
      std::stable_sort(bench_idx.begin(), bench_idx.end(), [&](int x, int y) { return pred[x] < pred[y]; });
      bench_idx.resize(top_k);
      std::sort(bench_idx.begin(), bench_idx.end());
      cands.clear();
      for (int i : bench_idx) cands.push_back(candidates[i]);
      if (ms_out)
        for (int i = 0; i < n_candidates; ++i) ms_out[i] = -1.0f;
    }
  }
  const int def = (G * 7) / 8;
  if (std::find(cands.begin(), cands.end(), def) == cands.end()) cands.push_back(def);
  auto call = [&](int gw) -> int {
    cfg.gemm_wgs = gw;
    switch (a->op) {
      case IRIS_OP_AG_MM:
        return iris_ag_mm(a->C, a->out, a->srcs, a->W, a->B, a->bias, a->M, a->N, a->K, &cfg, nullptr, 0, stream);
      case IRIS_OP_MM_RS:
        return iris_mm_rs_local(a->out, a->C, a->A, a->B, a->bias, a->srcs, a->W, a->rank, a->M, a->N, a->K, &cfg,
                                nullptr, 0, stream);
      case IRIS_OP_MM_AR:
        return iris_mm_ar_local(a->out, a->C, a->A, a->B, a->bias, a->srcs, a->W, a->M, a->N, a->K, &cfg, nullptr,
                                0, stream);
      case IRIS_OP_CONCURRENT:
        return iris_concurrent(a->C, a->A, a->B, a->bias, a->M, a->N, a->K,
                               a->collective > 0 ? a->collective : IRIS_COLL_ALL_REDUCE, a->rank, a->out, a->srcs,
                               a->W, a->comm_elems, &cfg, nullptr, 0, stream);
      case IRIS_OP_MM_AG:
        return iris_mm_ag_local(a->out, a->A, a->B, a->bias, a->srcs, a->W, a->rank, a->M, a->N, a->K, &cfg,
                                nullptr, 0, stream);
    }
    return fail(IRIS_ERR_INVALID_ARG, "unknown op %d", a->op);
  };
  hipEvent_t e0, e1;
  hipError_t he = hipEventCreate(&e0);
  if (he != hipSuccess) return hip_fail(he, "hipEventCreate");
  he = hipEventCreate(&e1);
  if (he != hipSuccess) {
    (void)hipEventDestroy(e0);
    return hip_fail(he, "hipEventCreate");
  }
  const hipStream_t s = (hipStream_t)stream;
  int best = -1;
  float best_ms = 0;
  int status = IRIS_OK;
  for (size_t i = 0; i < cands.size() && status == IRIS_OK; ++i) {
    const int gw = cands[i];
    for (int w = 0; w < 2 && status == IRIS_OK; ++w) status = call(gw);
    std::vector<float> t;
    for (int r = 0; r < reps && status == IRIS_OK; ++r) {
      he = hipEventRecord(e0, s);
      if (he != hipSuccess) { status = hip_fail(he, "hipEventRecord"); break; }
      status = call(gw);
      he = hipEventRecord(e1, s);
      if (he != hipSuccess) { status = hip_fail(he, "hipEventRecord"); break; }
      if (status) break;
      he = hipEventSynchronize(e1);
      if (he != hipSuccess) {
        status = hip_fail(he, "hipEventSynchronize");
        break;
      }
      float ms = 0;
      (void)hipEventElapsedTime(&ms, e0, e1);
      t.push_back(ms);
    }
    if (status) break;
    std::sort(t.begin(), t.end());
    const float med = t[t.size() / 2];
    if (ms_out && i < bench_idx.size()) ms_out[bench_idx[i]] = med;
    if (best < 0 || med < best_ms || (med == best_ms && gw > best)) {
      best = gw;
      best_ms = med;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (status) return status;
  *best_gemm_wgs = best;
  int dev;
  DevInfo di;
  if (current_device(&dev, &di) == IRIS_OK) {
    Resolved r{};
    resolve_static(&cfg, &r);
    // AG keys on K_local (args->K), the other ops on K, as run() looks them up
    const int coll = a->op == IRIS_OP_CONCURRENT ? (a->collective > 0 ? a->collective : IRIS_COLL_ALL_REDUCE) : 0;
    remember_gemm_wgs(cache_key(di.arch, a->op * 16 + coll, a->M, a->N, a->K, a->W, r.bm, r.bn, r.bk, r.gm), best);
  }
  return IRIS_OK;
}

int iris_last_windows(void* workspace, void* stream, double* gs_ns, double* ge_ns, double* cs_ns, double* ce_ns) {
  g_msg.clear();
  void* ws = workspace;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  LastLaunch last;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!ws) {
      auto it = g_ws.find({dev, stream});
      if (it == g_ws.end()) return fail(IRIS_ERR_INVALID_ARG, "no library workspace for this stream yet");
      ws = it->second.ptr;
    }
    auto lt = g_last.find(ws);
    if (lt == g_last.end()) return fail(IRIS_ERR_INVALID_ARG, "no launch recorded for this workspace");
    last = lt->second;
  }
  e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  std::vector<uint64_t> st((size_t)kMaxGrid * iris::kStampWords);
  e = hipMemcpy(st.data(), (char*)ws + last.stamp_off, st.size() * 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "stamp readback");
  DevInfo di;
  int d2;
  int s2 = current_device(&d2, &di);
  if (s2) return s2;
  uint64_t lo = ~0ull, gs = ~0ull, ge = 0, cs = ~0ull, ce = 0;
  for (int b = 0; b < last.grid; ++b) {
    const uint64_t* w = &st[(size_t)b * 4];
    if (w[1]) { gs = std::min(gs, w[0]); ge = std::max(ge, w[1]); }
    if (last.fused && w[3]) { cs = std::min(cs, w[2]); ce = std::max(ce, w[3]); }
  }
  for (int b = 0; b < last.comm_grid; ++b) {  // sequential mode: the comm kernel's own stamps
    const uint64_t* w = &st[(size_t)kMaxGrid * 4 + (size_t)b * 2];
    if (w[1]) { cs = std::min(cs, w[0]); ce = std::max(ce, w[1]); }
  }
  lo = std::min(gs, cs);
  const double ns_per_tick = 1e6 / (double)di.wall_khz;
  auto conv = [&](uint64_t v) { return (v == ~0ull || v == 0) ? -1.0 : (double)(v - lo) * ns_per_tick; };
  if (gs_ns) *gs_ns = conv(gs);
  if (ge_ns) *ge_ns = conv(ge);
  if (cs_ns) *cs_ns = conv(cs);
  if (ce_ns) *ce_ns = conv(ce);
  return IRIS_OK;
}

int iris_last_clock(void* workspace, void* stream, double* mhz) {
  g_msg.clear();
  if (!mhz) return fail(IRIS_ERR_INVALID_ARG, "mhz is NULL");
  *mhz = -1.0;
  void* ws = workspace;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  LastLaunch last;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!ws) {
      auto it = g_ws.find({dev, stream});
      if (it == g_ws.end()) return fail(IRIS_ERR_INVALID_ARG, "no library workspace for this stream yet");
      ws = it->second.ptr;
    }
    auto lt = g_last.find(ws);
    if (lt == g_last.end()) return fail(IRIS_ERR_INVALID_ARG, "no launch recorded for this workspace");
    last = lt->second;
  }
  e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  std::vector<uint64_t> ck((size_t)kMaxGrid * 4);
  e = hipMemcpy(ck.data(), (char*)ws + last.stamp_off + (size_t)kMaxGrid * iris::kClockOff * 8, ck.size() * 8,
                hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "clock readback");
  DevInfo di;
  int d2;
  int s2 = current_device(&d2, &di);
  if (s2) return s2;
  double cycles = 0, ticks = 0;
  for (int b = 0; b < last.grid; ++b) {
    const uint64_t* w = &ck[(size_t)b * 4];
    if (w[2] > w[0] && w[3] > w[1]) {
      cycles += (double)(w[2] - w[0]);
      ticks += (double)(w[3] - w[1]);
    }
  }
  if (ticks > 0) *mhz = cycles / ticks * (double)di.wall_khz / 1e3;
  return IRIS_OK;
}

int iris_mfma_ceiling(int32_t random_operands, int32_t iters, void* stream, double* tflops, double* clock_mhz) {
  g_msg.clear();
  if (!tflops || !clock_mhz) return fail(IRIS_ERR_INVALID_ARG, "tflops and clock_mhz must not be NULL");
  *tflops = -1.0;
  *clock_mhz = -1.0;
  if (iters < 1 || iters > (1 << 22)) return fail(IRIS_ERR_INVALID_ARG, "iters must be in [1, 2^22] (got %d)", iters);
  int dev = 0;
  DevInfo di;
  int st = current_device(&dev, &di);
  if (st) return st;
  const int grid = di.cus * 4;
  float ms = 0.0f;
  double cycles = 0.0, ticks = 0.0;
  const hipError_t e =
      iris::mfma_ceiling_run(random_operands != 0, iters, grid, (hipStream_t)stream, &ms, &cycles, &ticks);
  if (e != hipSuccess) return hip_fail(e, "MFMA ceiling launch");
  if (ms > 0.0f) *tflops = iris::kCeilingFlopPerTrip * (double)iters * (double)grid / ((double)ms * 1e-3) / 1e12;
  if (ticks > 0.0) *clock_mhz = cycles / ticks * (double)di.wall_khz / 1e3;
  return IRIS_OK;
}

int iris_check_device_error(void* workspace, void* stream) {
  g_msg.clear();
  if (workspace) {
    if ((uintptr_t)workspace % 256 != 0) return fail(IRIS_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
    return read_status(workspace, (hipStream_t)stream);
  }
  // the library's own workspace for this stream and the device's static
  // scratch (iris_ag_mm_noalloc), each if it has been used
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void* own = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_ws.find({dev, stream});
    if (it != g_ws.end()) own = it->second.ptr;
  }
  int status = IRIS_OK;
  for (void* ws : {own, iris::scratch_if_set_up(dev)}) {
    if (!ws) continue;
    const int st = read_status(ws, (hipStream_t)stream);
    if (st != IRIS_OK) status = st;
  }
  return status;
}

int iris_device_info(int32_t device, iris_device_info_t* info) {
  g_msg.clear();
  if (!info) return fail(IRIS_ERR_INVALID_ARG, "info is NULL");
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n == 0) return fail(IRIS_ERR_NO_DEVICE, "no HIP device");
  if (device < 0 || device >= n) return fail(IRIS_ERR_INVALID_ARG, "device %d out of range", device);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  memset(info, 0, sizeof *info);
  info->device = device;
  info->compute_units = prop.multiProcessorCount;
  info->clock_khz = prop.clockRate;
  info->memory_clock_khz = prop.memoryClockRate;
  info->lds_bytes_per_cu = (int32_t)prop.maxSharedMemoryPerMultiProcessor;
  info->global_mem_bytes = (int64_t)prop.totalGlobalMem;
  snprintf(info->arch, sizeof info->arch, "%s", prop.gcnArchName);
  const bool gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  info->peak_fp16_tflops = gfx950 ? (double)prop.multiProcessorCount * prop.clockRate * 1e3 * 4096.0 / 1e12 : 0.0;
  info->peak_hbm_gbps = gfx950 ? 8000.0 : 0.0;
  return IRIS_OK;
}

const char* iris_status_str(int32_t s) {
  switch (s) {
    case IRIS_OK: return "IRIS_OK";
    case IRIS_ERR_INVALID_ARG: return "IRIS_ERR_INVALID_ARG";
    case IRIS_ERR_UNSUPPORTED: return "IRIS_ERR_UNSUPPORTED";
    case IRIS_ERR_CONFIG: return "IRIS_ERR_CONFIG";
    case IRIS_ERR_ALIGNMENT: return "IRIS_ERR_ALIGNMENT";
    case IRIS_ERR_NO_MEMORY: return "IRIS_ERR_NO_MEMORY";
    case IRIS_ERR_HIP: return "IRIS_ERR_HIP";
    case IRIS_ERR_WORKSPACE: return "IRIS_ERR_WORKSPACE";
    case IRIS_ERR_NO_DEVICE: return "IRIS_ERR_NO_DEVICE";
    case IRIS_ERR_DEVICE_TIMEOUT: return "IRIS_ERR_DEVICE_TIMEOUT";
  }
  return "IRIS_ERR_UNKNOWN";
}

const char* iris_last_error_message(void) { return g_msg.c_str(); }

int iris_finalize(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int status = IRIS_OK;
  for (auto& kv : g_ws) {
    if (kv.second.ptr) {
      (void)hipSetDevice(kv.first.first);
      (void)hipStreamSynchronize((hipStream_t)kv.first.second);
      if (hipFree(kv.second.ptr) != hipSuccess) status = IRIS_ERR_HIP;
    }
  }
  g_ws.clear();
  g_last.clear();
  for (auto& kv : g_side) {
    (void)hipSetDevice(kv.first.first);
    if (kv.second.s && hipStreamSynchronize(kv.second.s) != hipSuccess) status = IRIS_ERR_HIP;
    if (kv.second.join) (void)hipEventDestroy(kv.second.join);
    if (kv.second.fork) (void)hipEventDestroy(kv.second.fork);
    if (kv.second.s && hipStreamDestroy(kv.second.s) != hipSuccess) status = IRIS_ERR_HIP;
  }
  g_side.clear();
  return status;
}

}  // extern "C"
