// libwsic C ABI: argument checks, workspace layout, the SIC pass driver and the rate
// controller. All arithmetic runs in the kernels of this library; this file only orders
// launches on the caller's stream and reads back scalars.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

// Scratch of the entry point that allocates nothing (wsic_distortion_noalloc): one copy per GPU,
// held until the process ends. Host code never uses the array's name as an address: the device
// address of each GPU's copy comes from hipGetSymbolAddress (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[WSIC_NOALLOC_SCRATCH_BYTES];

namespace wsic {

// ============================================================== error state
static thread_local char g_err[1024] = {0};

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}
void clear_error() { g_err[0] = 0; }
const char* last_error() { return g_err; }

// ============================================================== launch timing
namespace {
struct PendingEvent {
  std::string family;
  hipEvent_t a, b;
  double work;
};
struct ProfAcc {
  int64_t launches = 0;
  double ms = 0.0, work = 0.0;
};
bool g_prof = false;
std::vector<std::string> g_prof_only;  // families to time; empty = all
std::vector<PendingEvent> g_pending;
std::map<std::string, ProfAcc> g_acc;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

int prof_collect() {
  for (auto& p : g_pending) {
    if (!p.a || !p.b) continue;
    WSIC_HIP_TRY(hipEventSynchronize(p.b));
    float ms = 0.f;
    WSIC_HIP_TRY(hipEventElapsedTime(&ms, p.a, p.b));
    ProfAcc& acc = g_acc[p.family];
    acc.launches += 1;
    acc.ms += ms;
    acc.work += p.work;
    g_event_pool.push_back(p.a);
    g_event_pool.push_back(p.b);
  }
  g_pending.clear();
  return WSIC_OK;
}
}  // namespace

ProfToken prof_begin(const char* family) {
  if (!g_prof) return ProfToken{-1, nullptr, nullptr};
  if (!g_prof_only.empty()) {
    bool sel = false;
    for (const auto& f : g_prof_only) sel = sel || f == family;
    if (!sel) return ProfToken{-1, nullptr, nullptr};
  }
  PendingEvent p{family, pool_event(), pool_event(), 0.0};
  if (!p.a || !p.b) return ProfToken{-1, nullptr, nullptr};
  g_pending.push_back(p);
  return ProfToken{(int)g_pending.size() - 1, p.a, p.b};
}

void prof_end(ProfToken t, double work) {
  if (t.slot < 0 || t.slot >= (int)g_pending.size()) return;
  g_pending[t.slot].work = work;
}

// ============================================================== static scratch
namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

// Device address of the current device's copy of `scratch`, looked up once per device (with that
// device current) and kept.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("hipGetDevice failed: %s", hipGetErrorString(e));
    return WSIC_E_HIP;
  }
  if (dev < 0 || dev >= MAX_DEVICES) {
    set_error("device index %d out of range", dev);
    return WSIC_E_INVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("hipGetSymbolAddress of the static scratch failed on device %d: %s", dev,
                hipGetErrorString(e));
      return WSIC_E_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WSIC_OK;
}

// ============================================================== workspace layouts
namespace {

constexpr size_t FLAGS_BYTES = 256;
constexpr int BW = 128;  // SIC leaf width

struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base((char*)p) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

// int8 operand rows: padded to 64 bytes, padding kept zero
// int8 rows are padded to whole 128-byte lines (zeros): the products read whole K-steps, and the
// super-block product fetches whole lines
inline int64_t ld_i8(int64_t n_in) { return (n_in + 127) / 128 * 128; }

struct SicWs {
  int* flags;       // setup checks
  double* invd;
  double* Y;
  double* G;
  double* Bpk;
  // integer interference product
  double* escale;   // 2^(e_j - P)
  double* bscale;   // 2^e_j
  int8_t* D;        // LIMBS planes n_in x ld_i8
  int8_t* q8;       // n_out x ld_i8
  // per-pass state, cleared by one fill: flags word(s), row |q| sums, excess list counts
  int* pflags;      // [0] flag bits of the pass, [1] exact re-derivations, [2] re-checked decisions
  double* absq;
  int* ocnt;
  size_t pass_bytes;
  int2* olist;
};
SicWs carve_sic(Carve& cv, int64_t n_out, int64_t n_in) {
  SicWs w;
  w.flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
  w.invd = cv.take<double>((size_t)n_in);
  w.Y = cv.take<double>((size_t)n_out * n_in);
  w.G = cv.take<double>((size_t)n_out * n_in);
  w.Bpk = cv.take<double>((size_t)sic_pack_doubles(n_in));
  w.escale = cv.take<double>((size_t)n_in);
  w.bscale = cv.take<double>((size_t)n_in);
  w.D = cv.take<int8_t>((size_t)LIMBS * n_in * ld_i8(n_in));
  w.q8 = cv.take<int8_t>((size_t)n_out * ld_i8(n_in));
  // contiguous: flags, absq, ocnt (one fill per pass)
  const size_t off0 = cv.off;
  w.pflags = cv.take<int>(FLAGS_BYTES / sizeof(int));
  w.absq = (double*)(cv.base ? cv.base + cv.off : nullptr);
  cv.off += (size_t)n_out * sizeof(double);
  w.ocnt = (int*)(cv.base ? cv.base + cv.off : nullptr);
  cv.off = align_up(cv.off + (size_t)n_out * sizeof(int));
  w.pass_bytes = cv.off - off0;
  w.olist = cv.take<int2>((size_t)n_out * OCAP);
  return w;
}

struct HistWs {
  unsigned long long* bins;
  unsigned int* ovf_count;
  int32_t* ovf;
  EntropyResult* res;
};
HistWs carve_hist(Carve& cv) {
  HistWs h;
  // bins and the overflow counter are adjacent so one fill clears both
  h.bins = cv.take<unsigned long long>(HIST_BINS + 32);
  h.ovf_count = (unsigned int*)(h.bins ? h.bins + HIST_BINS : nullptr);
  h.ovf = cv.take<int32_t>(OVF_CAP);
  h.res = cv.take<EntropyResult>(1);
  return h;
}
constexpr size_t HIST_CLEAR_BYTES = (HIST_BINS + 32) * sizeof(unsigned long long);

// per-column histograms: bins (n_in x COL_BINS), overflow count right after them (one fill clears
// both), overflow list of (column, code), per-column sums and their total
struct ColHistWs {
  unsigned* bins;
  unsigned* ovf_count;
  int2* ovf;
  double* colS;
  double* out;
  int64_t n_in;
};
ColHistWs carve_colhist(Carve& cv, int64_t n_in) {
  ColHistWs h;
  h.bins = cv.take<unsigned>((size_t)n_in * COL_BINS + 64);
  h.ovf_count = h.bins ? h.bins + (size_t)n_in * COL_BINS : nullptr;
  h.ovf = cv.take<int2>(OVF_CAP);
  h.colS = cv.take<double>((size_t)n_in);
  h.out = cv.take<double>(1);
  h.n_in = n_in;
  return h;
}

// The secant controller's probe: PROBE_K grid scales tried at once on a layer of PROBE_K groups
// of probe_rows(n_out) evenly spaced rows (0: no probe for this shape). It reuses the pass
// buffers of the real layer, so it needs at most n_out rows. A pass is bound by the latency of
// its workgroups (16 rows each, one per CU) up to 4096 rows, so the probe's 4096 rows cost as
// much as a whole pass of a layer that small; it runs only where it costs at most a quarter of
// a pass. (On 4096- to 11008-row layers, measured with it: 34 passes over 6 targets against 32.)
constexpr int PROBE_K = PROBE_MAX;
constexpr int64_t PROBE_MIN_ROWS = 16384;
int probe_rows(int64_t n_out) {
  if (n_out < PROBE_MIN_ROWS) return 0;
  return 512;
}

struct WfWs {
  SicWs sic;
  int32_t* codes2;
  float* resid2;
  double* colvar;
  double* diag;
  HistWs hist;
  ColHistWs col;
  double* Yp;                  // the probe layer's Y (PROBE_K * probe_rows x n_in)
  unsigned long long* pbins;   // one histogram (and its overflow count) per probe group
  EntropyResult* pres;
};
constexpr size_t PROBE_BIN_STRIDE = HIST_BINS + 32;
WfWs carve_wf(Carve& cv, int64_t n_out, int64_t n_in) {
  WfWs w;
  w.sic = carve_sic(cv, n_out, n_in);
  w.codes2 = cv.take<int32_t>((size_t)n_out * n_in);
  w.resid2 = cv.take<float>((size_t)n_out * n_in);
  // column variances (n_in), then the partial sums from an even offset (16-byte aligned)
  w.colvar = cv.take<double>((size_t)colstats_doubles(n_out, n_in) + n_in + 1);
  w.diag = cv.take<double>((size_t)n_in);
  w.hist = carve_hist(cv);
  w.col = carve_colhist(cv, n_in);
  const int S = probe_rows(n_out);
  w.Yp = S ? cv.take<double>((size_t)PROBE_K * S * n_in) : nullptr;
  w.pbins = S ? cv.take<unsigned long long>(PROBE_K * PROBE_BIN_STRIDE) : nullptr;
  w.pres = S ? cv.take<EntropyResult>(PROBE_K) : nullptr;
  return w;
}

// partial sums written by k_dist_resid: one per 1024-column by DIST_ROWS-row tile
int64_t dist_resid_partials(int64_t n_out, int64_t n_in) {
  return ((n_in + 1023) / 1024) * ((n_out + DIST_ROWS - 1) / DIST_ROWS);
}
int64_t dist_partials(int64_t n_out, int64_t n_in) {
  const int64_t b = ((n_out + 63) / 64) * ((n_in + 63) / 64);  // direct mode: one per GEMM tile
  return std::max(dist_resid_partials(n_out, n_in), b);
}
struct DistWs {
  int* flags;
  double* invd;
  double* delta;
  double* partial;
  double* out;
};
DistWs carve_dist(Carve& cv, int64_t n_out, int64_t n_in) {
  DistWs d;
  d.flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
  d.invd = cv.take<double>((size_t)n_in);
  d.delta = cv.take<double>((size_t)n_in);
  d.partial = cv.take<double>((size_t)dist_partials(n_out, n_in));
  d.out = cv.take<double>(1);
  return d;
}

// SoftWater class scales s_r = sqrt(lambda_r) and their own check flag
struct ScaleWs {
  double* s;
  int* flags;
};
ScaleWs carve_scales(Carve& cv, int64_t n_out) {
  ScaleWs r;
  r.s = cv.take<double>((size_t)n_out);
  r.flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
  return r;
}

// softmax curvature of `rows` calibration inputs over K classes
struct CurvWs {
  int* flags;
  float* Lg;
  int64_t ldl;
  float2* part;
  float* rmax;
  double* rinvz;
  double* cpart;
};
CurvWs carve_curv(Carve& cv, int64_t rows, int64_t K) {
  int64_t ntn, nchunk, ldl;
  curvature_dims(rows, K, &ntn, &nchunk, &ldl);
  CurvWs c;
  c.flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
  c.Lg = cv.take<float>((size_t)rows * (size_t)ldl);
  c.ldl = ldl;
  c.part = cv.take<float2>((size_t)rows * (size_t)ntn);
  c.rmax = cv.take<float>((size_t)rows);
  c.rinvz = cv.take<double>((size_t)rows);
  c.cpart = cv.take<double>((size_t)nchunk * (size_t)K);
  return c;
}

constexpr int SUMSQ_BLOCKS = 1024;

// ---------------------------------------------------------------- rANS container layout
constexpr uint32_t RANS_MAGIC = 0x534E5257u, RANS_PROB = 14, RANS_M = 1u << RANS_PROB;
constexpr int RANS_WIN = 2047, RANS_MAX_SYM = 2 * RANS_WIN + 2;
inline size_t a16(size_t x) { return (x + 15) / 16 * 16; }
struct RansLayout {
  size_t freq, gofs, eofs, states, esc, payload, total;
};
RansLayout rans_layout(int64_t G, int64_t nsym, int64_t n_esc, int64_t nw) {
  RansLayout r;
  r.freq = 64;
  r.gofs = a16(r.freq + 2 * (size_t)nsym);
  r.eofs = a16(r.gofs + 4 * (size_t)(G + 1));
  r.states = a16(r.eofs + 4 * (size_t)(G + 1));
  r.esc = a16(r.states + 4 * 64 * (size_t)G);
  r.payload = a16(r.esc + 4 * (size_t)n_esc);
  r.total = r.payload + 2 * (size_t)nw;
  return r;
}
int64_t rans_groups(int64_t n, int64_t L) { return (n + 64 * L - 1) / (64 * L); }

// frequencies scaled to 2^14: max(1, floor(c M / N)) for every present symbol, the remainder to the
// most frequent symbol, an excess taken one by one from the largest frequency above 1 (lowest index
// first on ties)
std::vector<uint16_t> rans_normalize(const std::vector<int64_t>& counts, int64_t N) {
  const size_t n = counts.size();
  std::vector<int64_t> f(n, 0);
  int64_t sum = 0;
  for (size_t i = 0; i < n; ++i) {
    if (counts[i] > 0) f[i] = std::max<int64_t>(1, (counts[i] * (int64_t)RANS_M) / N);
    sum += f[i];
  }
  int64_t diff = (int64_t)RANS_M - sum;
  if (diff > 0) {
    size_t im = 0;
    for (size_t i = 1; i < n; ++i)
      if (counts[i] > counts[im]) im = i;
    f[im] += diff;
  }
  while (diff < 0) {
    size_t im = 0;
    int64_t best = -1;
    for (size_t i = 0; i < n; ++i)
      if (f[i] > 1 && f[i] > best) {
        best = f[i];
        im = i;
      }
    f[im] -= 1;
    ++diff;
  }
  std::vector<uint16_t> out(n);
  for (size_t i = 0; i < n; ++i) out[i] = (uint16_t)f[i];
  return out;
}

size_t ws_bytes_for(int op, int64_t n_out, int64_t n_in) {
  Carve cv(nullptr);
  switch (op) {
    case WSIC_OP_COVARIANCE:
      cv.take<int>(FLAGS_BYTES / sizeof(int));
      cv.take<char>(syrk_split_bytes(n_in));  // K-split of the launch's last partial round
      break;
    case WSIC_OP_CHOLESKY:
      cv.take<int>(FLAGS_BYTES / sizeof(int));
      cv.take<double>(2 * 64 * 64);  // two diagonal-block slots
      break;
    case WSIC_OP_SIC:
      carve_sic(cv, n_out, n_in);
      break;
    case WSIC_OP_WATERFILL:
      carve_wf(cv, n_out, n_in);
      break;
    case WSIC_OP_ENTROPY:
      cv.take<int>(FLAGS_BYTES / sizeof(int));
      carve_hist(cv);
      break;
    case WSIC_OP_DISTORTION:
      carve_dist(cv, n_out, n_in);
      break;
    case WSIC_OP_CURVATURE:
      carve_curv(cv, n_out, n_in);
      break;
    case WSIC_OP_ENTROPY_COLUMNS:
      cv.take<int>(FLAGS_BYTES / sizeof(int));
      carve_colhist(cv, n_in);
      break;
    case WSIC_OP_LMMSE:
      cv.take<int>(FLAGS_BYTES / sizeof(int));
      cv.take<double>((size_t)n_out * n_in);
      cv.take<double>(3 * (size_t)n_out + 2);
      break;
    case WSIC_OP_LIVE:
      cv.take<int>(FLAGS_BYTES / sizeof(int));
      cv.take<long long>(1);
      break;
    case WSIC_OP_RANS_ENC: {  // n_out = symbols per lane, n_in = number of codes
      const int64_t G = rans_groups(n_in, n_out);
      cv.take<int>(FLAGS_BYTES / sizeof(int));
      carve_hist(cv);
      cv.take<uint32_t>(2 * (size_t)G + 2);
      cv.take<uint16_t>((size_t)G * 64 * (size_t)n_out);
      break;
    }
    case WSIC_OP_RANS_DEC:  // n_in = columns of the layer (dequantization)
      cv.take<int>(FLAGS_BYTES / sizeof(int));
      cv.take<double>((size_t)n_in);
      break;
    case WSIC_OP_GAUSS_RATE:
      cv.take<int>(FLAGS_BYTES / sizeof(int));
      cv.take<double>(SUMSQ_BLOCKS + 2);
      cv.take<double>((size_t)n_in);
      break;
    case WSIC_OP_SOFTWATER:
      carve_wf(cv, n_out, n_in);
      carve_scales(cv, n_out);
      break;
    case WSIC_OP_SOFTWATER_DIST:
      carve_dist(cv, n_out, n_in);
      carve_scales(cv, n_out);
      break;
    default:
      return 0;
  }
  return cv.off;
}

// ============================================================== checks
int check_ws(int op, int64_t n_out, int64_t n_in, void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(op, n_out, n_in);
  if (!ws || ws_bytes < need) {
    set_error("workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
    return WSIC_E_WORKSPACE;
  }
  if (((uintptr_t)ws) % 256 != 0) {
    set_error("workspace must be 256-byte aligned");
    return WSIC_E_INVAL;
  }
  return WSIC_OK;
}

int check_layer(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw) {
  if (!W) {
    set_error("W is null");
    return WSIC_E_INVAL;
  }
  if (dtype != WSIC_F32 && dtype != WSIC_BF16) {
    set_error("unknown dtype %d", dtype);
    return WSIC_E_INVAL;
  }
  if (n_out <= 0 || n_in <= 0 || ldw < n_in) {
    set_error("bad layer shape n_out=%lld n_in=%lld ldw=%lld", (long long)n_out, (long long)n_in,
              (long long)ldw);
    return WSIC_E_INVAL;
  }
  if (n_in > (int64_t)1 << 20 || n_out > (int64_t)1 << 28) {
    set_error("layer too large");
    return WSIC_E_INVAL;
  }
  return WSIC_OK;
}

#define WSIC_TRY(expr)         \
  do {                         \
    int _rc = (expr);          \
    if (_rc != WSIC_OK) return _rc; \
  } while (0)

// Device -> host reads at the synchronization points of the API. The pieces land in a pinned
// per-thread staging buffer (a direct DMA target, unlike pageable memory) and completion is
// polled on an event, which returns sooner than a blocking stream synchronization; after a
// short spin the wait blocks on the event instead.
struct ReadPiece {
  void* host;
  const void* dev;
  size_t bytes;
};

struct HostStage {
  char* buf = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
};
thread_local HostStage t_stage;  // never freed: one small pinned buffer per calling thread

// Copies to the calling thread's pinned staging buffer are enqueued and an event recorded
// (read_back_start); read_back_finish polls the event and copies out. One read-back per thread
// at a time.
int read_back_start(const ReadPiece* p, int n, hipStream_t st) {
  size_t total = 0;
  for (int i = 0; i < n; ++i) total += align_up(p[i].bytes, 16);
  HostStage& hs = t_stage;
  if (!hs.ev) WSIC_HIP_TRY(hipEventCreateWithFlags(&hs.ev, hipEventDisableTiming));
  if (total > hs.cap) {
    const size_t cap = std::max<size_t>(total, 4096);
    char* nb = nullptr;
    WSIC_HIP_TRY(hipHostMalloc((void**)&nb, cap, hipHostMallocDefault));
    if (hs.buf) (void)hipHostFree(hs.buf);
    hs.buf = nb;
    hs.cap = cap;
  }
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    WSIC_HIP_TRY(hipMemcpyAsync(hs.buf + off, p[i].dev, p[i].bytes, hipMemcpyDeviceToHost, st));
    off += align_up(p[i].bytes, 16);
  }
  WSIC_HIP_TRY(hipEventRecord(hs.ev, st));
  return WSIC_OK;
}

int read_back_finish(const ReadPiece* p, int n) {
  HostStage& hs = t_stage;
  hipError_t e = hipErrorNotReady;
  for (int spin = 0; spin < (1 << 22) && e == hipErrorNotReady; ++spin) e = hipEventQuery(hs.ev);
  if (e == hipErrorNotReady) e = hipEventSynchronize(hs.ev);
  if (e != hipSuccess) {
    set_error("device read-back failed: %s", hipGetErrorString(e));
    return WSIC_E_HIP;
  }
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    std::memcpy(p[i].host, hs.buf + off, p[i].bytes);
    off += align_up(p[i].bytes, 16);
  }
  return WSIC_OK;
}

int read_back(const ReadPiece* p, int n, hipStream_t st) {
  WSIC_TRY(read_back_start(p, n, st));
  return read_back_finish(p, n);
}

int read_flags(const int* dflags, int* out, hipStream_t st) {
  const ReadPiece pc{out, dflags, sizeof(int)};
  return read_back(&pc, 1, st);
}

int flags_status(int f, const char* what) {
  if (f & FLAG_NONFINITE) {
    set_error("%s: NaN or Inf in an input", what);
    return WSIC_E_NONFINITE;
  }
  if (f & FLAG_BAD_SCALE) {
    set_error("%s: a class curvature is not positive and finite", what);
    return WSIC_E_INVAL;
  }
  if (f & FLAG_BAD_DIAG) {
    set_error("%s: U has a diagonal entry that is not positive and finite", what);
    return WSIC_E_INVAL;
  }
  if (f & FLAG_RANGE) {
    set_error("%s: a code does not fit int32 (grid scale too small)", what);
    return WSIC_E_RANGE;
  }
  return WSIC_OK;
}

// ============================================================== SIC pass
struct SicCtx {
  int64_t n_out, n_in;
  const void* W;
  int dtype;
  int64_t ldw;
  const double* U;
  int64_t ldu;
  SicWs ws;
  hipStream_t st;
  bool i8;             // interference by the exact int8 limb product (else fp64 MFMA)
  double guard_scale;  // multiplies the error bound (testing hook; 1 in normal use)
  bool super_launch;   // int8 mode: a range of up to SUPER blocks in one launch (else per block)
  const double* rs;    // class scales: row r of Y = W U^T is multiplied by rs[r] (nullable)
};

// diagnostic switches (wsic_debug_set): alternative paths with the same results
struct DebugKnobs {
  std::atomic<bool> fp64_product{false};
  std::atomic<bool> super_blocks{true};
  std::atomic<double> guard_scale{1.0};
  std::atomic<bool> chol_fused{true};
  std::atomic<bool> logits_generic{false};
  std::atomic<bool> trace{false};
  std::atomic<bool> probe{true};
};
DebugKnobs g_dbg;

SicCtx make_ctx(int64_t n_out, int64_t n_in, const void* W, int dtype, int64_t ldw,
                const double* U, int64_t ldu, const SicWs& ws, hipStream_t st) {
  SicCtx x{n_out, n_in, W, dtype, ldw, U, ldu, ws, st, true, 1.0, true, nullptr};
  x.i8 = !g_dbg.fp64_product.load();
  x.super_launch = g_dbg.super_blocks.load();
  x.guard_scale = g_dbg.guard_scale.load();
  return x;
}

// invd, Y = W U^T, input checks. Leaves flags on the device (read by the caller).
// With read_now false the flags stay on the device for the caller to read with its next read-back.
int sic_setup(const SicCtx& x, bool read_now = true) {
  WSIC_TRY(launch_fill_zero(x.ws.flags, FLAGS_BYTES, x.st));
  WSIC_TRY(launch_check_finite(x.W, x.dtype, x.n_out, x.n_in, x.ldw, x.ws.flags, x.st));
  WSIC_TRY(launch_prep(x.U, x.ldu, x.n_in, x.ws.invd, x.ws.flags, x.st));
  WSIC_TRY(launch_pack_blocks(x.U, x.ldu, x.n_in, x.ws.invd, x.ws.Bpk, x.st));
  if (x.i8) {
    WSIC_TRY(launch_limb_pack(x.U, x.ldu, x.n_in, x.ws.invd, x.ws.escale, x.ws.bscale, x.ws.D,
                              ld_i8(x.n_in), x.st));
    WSIC_TRY(launch_fill_zero(x.ws.q8, (size_t)x.n_out * ld_i8(x.n_in), x.st));
  }
  const double work = (double)x.n_out * (double)x.n_in * (double)(x.n_in + 1);
  WSIC_TRY(launch_gemm_y(x.dtype, x.n_out, x.n_in, x.n_in, x.W, x.ldw, x.U, x.ldu, x.ws.Y, x.n_in,
                         work, x.st));
  // class-aware grids c / (s_r U_jj) are the plain grids of the rows s_r w_r, whose Y rows are
  // s_r times those of w_r (SoftWater page, §2 "Aproximação Tratável")
  if (x.rs) WSIC_TRY(launch_scale_rows(x.ws.Y, x.n_out, x.n_in, x.n_in, x.rs, x.st));
  if (!read_now) return WSIC_OK;
  int f = 0;
  WSIC_TRY(read_flags(x.ws.flags, &f, x.st));
  return flags_status(f, "sic");
}

// Columns [lo, hi): G[:, lo:hi] holds the interference of every column >= hi (none when
// hi == n_in). Right half first, then its interference on the left half, then the left half.
// With the int8 product, a range of at most SUPER blocks is finished right to left by one
// launch that forms the interference of the range's finished columns itself (or, per block,
// by one leaf launch each when super_launch is off).
constexpr int64_t SUPER = 4;

// the leaf / super-block arguments shared by every launch of a pass over columns [j0, j0 + w)
LeafArgs leaf_args(const SicCtx& x, int64_t j0, int64_t w, bool has_g, double c, int32_t* codes,
                   int64_t ldq, float* resid, int64_t ldr) {
  LeafArgs a{};
  a.n_out = x.n_out;
  a.n_in = x.n_in;
  a.j0 = j0;
  a.w = (int)w;
  a.Y = x.ws.Y;
  a.ldy = x.n_in;
  a.G = has_g ? x.ws.G : nullptr;
  a.ldg = x.n_in;
  a.Bpk = x.ws.Bpk;
  a.invd = x.ws.invd;
  a.c = c;
  a.codes = codes;
  a.ldq = ldq;
  a.resid = resid;
  a.ldr = ldr;
  a.flags = x.ws.pflags;
  a.U = x.U;
  a.ldu = x.ldu;
  a.bscale = x.ws.bscale;
  a.guard_scale = x.guard_scale;
  a.q8 = x.ws.q8;
  a.ldq8 = ld_i8(x.n_in);
  a.absq = x.ws.absq;
  a.ocnt = x.ws.ocnt;
  a.olist = x.ws.olist;
  a.w_bytes = x.dtype == WSIC_BF16 ? 2 : 4;
  return a;
}

int sic_leaf_at(const SicCtx& x, int64_t j0, int64_t wb, int64_t hi, double c, int32_t* codes,
                int64_t ldq, float* resid, int64_t ldr, bool fuse) {
  LeafArgs a = leaf_args(x, j0, wb, hi < x.n_in, c, codes, ldq, resid, ldr);
  if (fuse && j0 + BW < hi) {
    a.D = x.ws.D;
    a.ldd = ld_i8(x.n_in);
    a.plane = x.n_in * a.ldd;
    a.escale = x.ws.escale;
    a.kf0 = j0 + BW;
    a.kf = (int)(hi - (j0 + BW));
  }
  return launch_sic_leaf(a, x.i8, x.st);
}

int sic_range(const SicCtx& x, int64_t lo, int64_t hi, double c, int32_t* codes, int64_t ldq,
              float* resid, int64_t ldr) {
  const int64_t w = hi - lo;
  const bool has_g = hi < x.n_in;
  if (x.i8 && w <= SUPER * BW && x.super_launch) {
    LeafArgs a = leaf_args(x, lo, w, has_g, c, codes, ldq, resid, ldr);
    a.D = x.ws.D;
    a.ldd = ld_i8(x.n_in);
    a.plane = x.n_in * a.ldd;
    a.escale = x.ws.escale;
    return launch_sic_super(a, x.st);
  }
  if (x.i8 && w <= SUPER * BW) {
    const int64_t nb = (w + BW - 1) / BW;
    for (int64_t b = nb - 1; b >= 0; --b) {
      const int64_t j0 = lo + b * BW;
      WSIC_TRY(sic_leaf_at(x, j0, std::min<int64_t>(BW, hi - j0), hi, c, codes, ldq, resid, ldr,
                           true));
    }
    return WSIC_OK;
  }
  if (w <= BW) return launch_sic_leaf(leaf_args(x, lo, w, has_g, c, codes, ldq, resid, ldr), x.i8, x.st);
  const int64_t nblk = (w + BW - 1) / BW;
  const int64_t mid = lo + BW * ((nblk + 1) / 2);
  WSIC_TRY(sic_range(x, mid, hi, c, codes, ldq, resid, ldr));
  if (x.i8) {
    const int64_t ld8 = ld_i8(x.n_in);
    WSIC_TRY(launch_gemm_i8(x.n_out, mid - lo, hi - mid, x.ws.q8 + mid, ld8, x.ws.D + lo * ld8 + mid,
                            ld8, x.n_in * ld8, x.ws.escale + lo, x.ws.G + lo, x.n_in,
                            has_g ? 1.0 : 0.0, x.st));
    return sic_range(x, lo, mid, c, codes, ldq, resid, ldr);
  }
  GemmArgs g{};
  g.M = x.n_out;
  g.N = mid - lo;
  g.K = hi - mid;
  g.A = codes + mid;
  g.lda = ldq;
  g.vec = x.ws.invd + mid;
  g.B = x.U + lo * x.ldu + mid;
  g.ldb = x.ldu;
  g.C = x.ws.G + lo;
  g.ldc = x.n_in;
  g.alpha = 1.0;
  g.beta = has_g ? 1.0 : 0.0;
  const double work = 2.0 * (double)g.M * (double)g.N * (double)g.K;
  WSIC_TRY(launch_gemm(A_CODES, EPI_STORE, g, "gemm_trail", work, x.st));
  return sic_range(x, lo, mid, c, codes, ldq, resid, ldr);
}

// One pass. With the int8 product, a row whose list of large codes overflows sends the whole
// pass through the fp64 product instead (the flag is read back with the pass's result).
int sic_pass_once(const SicCtx& x, double c, int32_t* codes, int64_t ldq, float* resid,
                  int64_t ldr) {
  WSIC_TRY(launch_fill_zero(x.ws.pflags, x.ws.pass_bytes, x.st));
  return sic_range(x, 0, x.n_in, c, codes, ldq, resid, ldr);
}

int sic_pass(const SicCtx& x, double c, int32_t* codes, int64_t ldq, float* resid, int64_t ldr,
             int* pass_flags) {
  WSIC_TRY(sic_pass_once(x, c, codes, ldq, resid, ldr));
  int f[3] = {0, 0, 0};
  const ReadPiece pc{f, x.ws.pflags, sizeof f};
  WSIC_TRY(read_back(&pc, 1, x.st));
  if (x.i8 && (f[0] & FLAG_OVERFLOW_LIST)) {
    SicCtx y = x;
    y.i8 = false;
    WSIC_TRY(sic_pass_once(y, c, codes, ldq, resid, ldr));
    WSIC_TRY(read_back(&pc, 1, x.st));
  }
  if (g_dbg.trace.load() && (f[1] || f[2]))
    std::fprintf(stderr, "wsic sic pass: %d decision(s) re-checked, %d workgroup(s) re-derived\n",
                 f[2], f[1]);
  if (pass_flags) *pass_flags = f[0];
  return flags_status(f[0], "sic pass");
}

// ============================================================== entropy
// Rate model for the controller's first two steps: column j's targets in grid units taken as
// N(0, (g_j / c)^2) with g_j = std(W column j) U_jj (the high-rate reading of WaterSIC's equal
// per-column distortion), rounded to integers and pooled over the columns. The pooled entropy of
// that mixture follows the measured H(c) of SIC codes much more closely in slope than the
// high-rate law (slope -1), which ignores both the low-rate shape and the spread of the g_j.
// g holds a few dozen quantiles of the g_j.
// With pooled == false the model is the mean of the per-column entropies instead (the rate of
// per-column entropy coding).
double gauss_col_entropy(const std::vector<double>& g, double c);
double gauss_mix_entropy(const std::vector<double>& g, double c, bool pooled = true) {
  if (!pooled) return gauss_col_entropy(g, c);
  double smax = 0.0;
  for (double v : g) smax = std::max(smax, v / c);
  const int Q = (int)std::ceil(6.0 * smax) + 1;
  std::vector<double> P(2 * Q + 1, 0.0);
  for (double gv : g) {
    const double sd = gv / c;
    if (!(sd > 0.0)) {
      P[Q] += 1.0;
      continue;
    }
    const double k = -1.0 / (sd * M_SQRT2);
    double lo = 0.5 * std::erfc(k * (-Q - 0.5));  // Phi((q - 1/2) / sd) for q = -Q
    for (int q = -Q; q <= Q; ++q) {
      const double hi = 0.5 * std::erfc(k * (q + 0.5));
      P[q + Q] += hi - lo;
      lo = hi;
    }
  }
  double h = 0.0;
  const double inv = 1.0 / (double)g.size();
  for (double v : P) {
    const double pv = v * inv;
    if (pv > 0.0) h -= pv * std::log2(pv);
  }
  return h;
}

double gauss_col_entropy(const std::vector<double>& g, double c) {
  double hsum = 0.0;
  for (double gv : g) hsum += gauss_mix_entropy(std::vector<double>{gv}, c, true);
  return hsum / (double)g.size();
}

std::vector<double> scale_quantiles(const std::vector<double>& var, const std::vector<double>& diag) {
  std::vector<double> g(var.size());
  for (size_t j = 0; j < var.size(); ++j) g[j] = std::sqrt(std::max(var[j], 0.0)) * std::fabs(diag[j]);
  std::sort(g.begin(), g.end());
  constexpr int NQ = 48;
  std::vector<double> q(NQ);
  for (int i = 0; i < NQ; ++i) q[i] = g[std::min(g.size() - 1, (size_t)((i + 0.5) / NQ * g.size()))];
  return q;
}

// log2 c with model entropy R (secant on log2 c from x0, a few steps)
double model_solve(const std::vector<double>& g, double R, double x0, bool pooled = true) {
  double xa = x0, ha = gauss_mix_entropy(g, std::exp2(xa), pooled);
  double slope = -1.0;
  for (int it = 0; it < 8 && std::fabs(ha - R) > 1e-4; ++it) {
    const double xb = xa + std::min(2.0, std::max(-2.0, (R - ha) / slope));
    const double hb = gauss_mix_entropy(g, std::exp2(xb), pooled);
    if (xb != xa) {
      const double sl = (hb - ha) / (xb - xa);
      if (sl < -0.25 && sl > -4.0) slope = sl;
    }
    xa = xb;
    ha = hb;
  }
  return xa;
}

int entropy_of(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq, const HistWs& h,
               const int* dflags, hipStream_t st, double* H, int64_t* nsym, int* flags_out,
               int* aux_out = nullptr, int* aux2_out = nullptr) {
  WSIC_TRY(launch_fill_zero(h.bins, HIST_CLEAR_BYTES, st));
  WSIC_TRY(launch_hist(codes, n_out, n_in, ldq, h.bins, h.ovf, h.ovf_count, st));
  WSIC_TRY(launch_entropy_reduce(h.bins, h.ovf_count, dflags, h.res, st));
  EntropyResult r;
  const ReadPiece pr{&r, h.res, sizeof r};
  WSIC_TRY(read_back(&pr, 1, st));
  if (flags_out) *flags_out = r.flags;
  if (aux_out) *aux_out = r.aux;
  if (aux2_out) *aux2_out = r.aux2;
  double s = r.sum_nlogn;
  int64_t ns = (int64_t)r.nsym;
  if (r.ovf_count > 0) {
    if (r.ovf_count > OVF_CAP) {
      set_error("entropy: %u codes beyond +-%d exceed the overflow list (%u)", r.ovf_count,
                HIST_HALF, OVF_CAP);
      return WSIC_E_RANGE;
    }
    std::vector<int32_t> v(r.ovf_count);
    const ReadPiece po{v.data(), h.ovf, v.size() * sizeof(int32_t)};
    WSIC_TRY(read_back(&po, 1, st));
    std::sort(v.begin(), v.end());
    size_t i = 0;
    while (i < v.size()) {
      size_t j = i;
      while (j < v.size() && v[j] == v[i]) ++j;
      const double cnt = (double)(j - i);
      s += cnt * std::log2(cnt);
      ++ns;
      i = j;
    }
  }
  const double N = (double)n_out * (double)n_in;
  *H = std::log2(N) - s / N;
  if (nsym) *nsym = ns;
  return WSIC_OK;
}

// Mean over columns of the column entropies: log2(n_out) - (sum_j S_j + overflow terms) / N.
// dflags (nullable): the SIC pass's three flag words, read back with the result.
int entropy_cols_of(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                    const ColHistWs& h, const int* dflags, hipStream_t st, double* H,
                    int* flags_out = nullptr, int* aux_out = nullptr, int* aux2_out = nullptr) {
  WSIC_TRY(launch_fill_zero(h.bins, ((size_t)n_in * COL_BINS + 64) * sizeof(unsigned), st));
  WSIC_TRY(launch_hist_cols(codes, n_out, n_in, ldq, h.bins, h.ovf, h.ovf_count, st));
  WSIC_TRY(launch_col_entropy(h.bins, n_in, h.colS, st));
  WSIC_TRY(launch_sum_partials(h.colS, n_in, h.out, st));
  double S = 0.0;
  unsigned novf = 0;
  int f[3] = {0, 0, 0};
  ReadPiece pr[3] = {{&S, h.out, sizeof(double)}, {&novf, h.ovf_count, sizeof(unsigned)},
                     {f, dflags, sizeof f}};
  WSIC_TRY(read_back(pr, dflags ? 3 : 2, st));
  if (flags_out) *flags_out = f[0];
  if (aux_out) *aux_out = f[1];
  if (aux2_out) *aux2_out = f[2];
  if (novf > 0) {
    if (novf > OVF_CAP) {
      set_error("entropy_columns: %u codes beyond +-%d exceed the overflow list (%u)", novf, COL_HALF,
                OVF_CAP);
      return WSIC_E_RANGE;
    }
    std::vector<int2> v(novf);
    const ReadPiece po{v.data(), h.ovf, v.size() * sizeof(int2)};
    WSIC_TRY(read_back(&po, 1, st));
    std::sort(v.begin(), v.end(), [](int2 a, int2 b) { return a.x != b.x ? a.x < b.x : a.y < b.y; });
    size_t i = 0;
    while (i < v.size()) {
      size_t k = i;
      while (k < v.size() && v[k].x == v[i].x && v[k].y == v[i].y) ++k;
      const double cnt = (double)(k - i);
      S += cnt * std::log2(cnt);
      i = k;
    }
  }
  *H = std::log2((double)n_out) - S / ((double)n_out * (double)n_in);
  return WSIC_OK;
}

}  // namespace
}  // namespace wsic

using namespace wsic;

// ============================================================== C ABI
extern "C" {

int wsic_version(void) { return WSIC_VERSION; }

int wsic_debug_set(int knob, double v) {
  using wsic::g_dbg;
  wsic::clear_error();
  if (!std::isfinite(v)) {
    wsic::set_error("debug_set: value is not finite");
    return WSIC_E_INVAL;
  }
  const bool on = v != 0.0;
  switch (knob) {
    case WSIC_DBG_FP64_PRODUCT: g_dbg.fp64_product = on; return WSIC_OK;
    case WSIC_DBG_SUPER_BLOCKS: g_dbg.super_blocks = on; return WSIC_OK;
    case WSIC_DBG_GUARD_SCALE:
      if (!(v >= 1.0)) {
        wsic::set_error("debug_set: guard scale %g below 1 would weaken the exact re-check", v);
        return WSIC_E_INVAL;
      }
      g_dbg.guard_scale = v;
      return WSIC_OK;
    case WSIC_DBG_CHOL_FUSED: g_dbg.chol_fused = on; return WSIC_OK;
    case WSIC_DBG_LOGITS_GENERIC: g_dbg.logits_generic = on; return WSIC_OK;
    case WSIC_DBG_TRACE: g_dbg.trace = on; return WSIC_OK;
    case WSIC_DBG_PROBE: g_dbg.probe = on; return WSIC_OK;
    default:
      wsic::set_error("debug_set: unknown knob %d", knob);
      return WSIC_E_INVAL;
  }
}

int wsic_debug_get(int knob, double* v) {
  using wsic::g_dbg;
  wsic::clear_error();
  if (!v) {
    wsic::set_error("debug_get: value pointer is null");
    return WSIC_E_INVAL;
  }
  switch (knob) {
    case WSIC_DBG_FP64_PRODUCT: *v = g_dbg.fp64_product.load(); return WSIC_OK;
    case WSIC_DBG_SUPER_BLOCKS: *v = g_dbg.super_blocks.load(); return WSIC_OK;
    case WSIC_DBG_GUARD_SCALE: *v = g_dbg.guard_scale.load(); return WSIC_OK;
    case WSIC_DBG_CHOL_FUSED: *v = g_dbg.chol_fused.load(); return WSIC_OK;
    case WSIC_DBG_LOGITS_GENERIC: *v = g_dbg.logits_generic.load(); return WSIC_OK;
    case WSIC_DBG_TRACE: *v = g_dbg.trace.load(); return WSIC_OK;
    case WSIC_DBG_PROBE: *v = g_dbg.probe.load(); return WSIC_OK;
    default:
      wsic::set_error("debug_get: unknown knob %d", knob);
      return WSIC_E_INVAL;
  }
}

void wsic_debug_reset(void) {
  using wsic::g_dbg;
  g_dbg.fp64_product = false;
  g_dbg.super_blocks = true;
  g_dbg.guard_scale = 1.0;
  g_dbg.chol_fused = true;
  g_dbg.logits_generic = false;
  g_dbg.trace = false;
  g_dbg.probe = true;
}

const char* wsic_last_error(void) { return wsic::last_error(); }

const char* wsic_status_str(int s) {
  switch (s) {
    case WSIC_OK: return "WSIC_OK";
    case WSIC_E_INVAL: return "WSIC_E_INVAL";
    case WSIC_E_NOT_PD: return "WSIC_E_NOT_PD";
    case WSIC_E_NONFINITE: return "WSIC_E_NONFINITE";
    case WSIC_E_NO_BRACKET: return "WSIC_E_NO_BRACKET";
    case WSIC_E_RANGE: return "WSIC_E_RANGE";
    case WSIC_E_WORKSPACE: return "WSIC_E_WORKSPACE";
    case WSIC_E_HIP: return "WSIC_E_HIP";
    default: return "WSIC_E_UNKNOWN";
  }
}

size_t wsic_workspace_bytes(int op, int64_t n_out, int64_t n_in) {
  if (n_in <= 0 ||
      (op != WSIC_OP_COVARIANCE && op != WSIC_OP_CHOLESKY && op != WSIC_OP_LIVE && op != WSIC_OP_RANS_DEC &&
       n_out <= 0))
    return 0;
  return ws_bytes_for(op, n_out, n_in);
}

int wsic_covariance(const void* X, int dtype, int64_t rows, int64_t n_in, int64_t ldx,
                    double alpha, double beta, double* Sigma, int64_t lds, void* ws,
                    size_t ws_bytes, void* stream) {
  try {
    clear_error();
    if (!X || !Sigma || rows <= 0 || n_in <= 0 || ldx < n_in || lds < n_in ||
        (dtype != WSIC_F32 && dtype != WSIC_BF16) || !std::isfinite(alpha) || !std::isfinite(beta)) {
      set_error("covariance: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_COVARIANCE, 0, n_in, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    int* flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
    const size_t split_bytes = syrk_split_bytes(n_in);
    void* split_ws = cv.take<char>(split_bytes);
    WSIC_TRY(launch_fill_zero(flags, FLAGS_BYTES, st));
    WSIC_TRY(launch_syrk(X, dtype, rows, n_in, ldx, alpha, beta, Sigma, lds, split_ws, split_bytes,
                         st));
    WSIC_TRY(launch_mirror_upper(Sigma, n_in, lds, st));
    WSIC_TRY(launch_diag_check(Sigma, n_in, lds, flags, st));
    int f = 0;
    WSIC_TRY(read_flags(flags, &f, st));
    return flags_status(f, "covariance");
  } catch (...) {
    set_error("covariance: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_cholesky(double* A, int64_t n, int64_t lda, int64_t* info, void* ws, size_t ws_bytes,
                  void* stream) {
  try {
    clear_error();
    if (!A || !info || n <= 0 || lda < n) {
      set_error("cholesky: bad argument");
      return WSIC_E_INVAL;
    }
    *info = 0;
    WSIC_TRY(check_ws(WSIC_OP_CHOLESKY, 0, n, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    int64_t* dinfo = cv.take<int64_t>(FLAGS_BYTES / sizeof(int64_t));
    double* slot[2];
    slot[0] = cv.take<double>(64 * 64);
    slot[1] = cv.take<double>(64 * 64);
    WSIC_TRY(launch_fill_zero(dinfo, FLAGS_BYTES, st));
    constexpr int NBK = 64;
    // diagnostic switch: update and next panel as separate launches
    const bool fused = g_dbg.chol_fused.load();
    // a panel's diagonal block lands in slot[step & 1] and is moved into A afterwards
    int64_t step = 0;
    WSIC_TRY(launch_potrf_panel(A, lda, 0, (int)std::min<int64_t>(NBK, n), n, dinfo, slot[0], st));
    for (int64_t kb = 0; kb + NBK < n; kb += NBK, ++step) {
      const int nbk = NBK;
      const int64_t m = n - kb - nbk;
      double* cur = slot[step & 1];
      double* next = slot[(step + 1) & 1];
      if (fused && chol_step_ok(A, lda, kb + nbk)) {
        // this step's trailing update and the next panel in one launch (which also moves this
        // step's diagonal block into A)
        WSIC_TRY(launch_chol_step(A, lda, kb, n, dinfo, cur, next, st));
        continue;
      }
      WSIC_TRY(launch_put_diag(A, lda, kb, nbk, cur, st));
      GemmArgs g{};
      g.M = m;
      g.N = m;
      g.K = nbk;
      g.A = A + kb * lda + kb + nbk;
      g.lda = lda;
      g.B = A + kb * lda + kb + nbk;
      g.ldb = lda;
      g.C = A + (kb + nbk) * lda + kb + nbk;
      g.ldc = lda;
      g.alpha = -1.0;
      g.beta = 1.0;
      g.upper_only = 1;
      const double work = (double)m * (double)(m + 1) * (double)nbk;
      WSIC_TRY(launch_gemm(A_F64_T, EPI_STORE, g, "gemm_chol", work, st));
      WSIC_TRY(launch_potrf_panel(A, lda, kb + nbk, (int)std::min<int64_t>(NBK, m), n, dinfo, next,
                                  st));
    }
    {  // the last panel's diagonal block
      const int64_t kb = step * NBK;
      WSIC_TRY(launch_put_diag(A, lda, kb, (int)(n - kb), slot[step & 1], st));
    }
    WSIC_TRY(launch_zero_lower(A, n, lda, st));
    const ReadPiece pi{info, dinfo, sizeof(int64_t)};
    WSIC_TRY(read_back(&pi, 1, st));
    if (*info != 0) {
      set_error("cholesky: leading minor %lld is not positive definite", (long long)*info);
      return WSIC_E_NOT_PD;
    }
    return WSIC_OK;
  } catch (...) {
    set_error("cholesky: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_sic_quantize(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                      const double* U, int64_t ldu, double c, int32_t* codes, int64_t ldq,
                      float* resid, int64_t ldr, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    WSIC_TRY(check_layer(W, dtype, n_out, n_in, ldw));
    if (!U || ldu < n_in || !codes || ldq < n_in || (resid && ldr < n_in) || !(c > 0.0) ||
        !std::isfinite(c)) {
      set_error("sic_quantize: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_SIC, n_out, n_in, ws, ws_bytes));
    Carve cv(ws);
    SicCtx x = make_ctx(n_out, n_in, W, dtype, ldw, U, ldu, carve_sic(cv, n_out, n_in),
                        (hipStream_t)stream);
    WSIC_TRY(sic_setup(x));
    return sic_pass(x, c, codes, ldq, resid, ldr, nullptr);
  } catch (...) {
    set_error("sic_quantize: internal exception");
    return WSIC_E_INVAL;
  }
}

// The rate controller over SIC passes; lam (nullable) gives SoftWater's class curvatures.
static int waterfill_run(const double* lam, const void* W, int dtype, int64_t n_out, int64_t n_in,
                         int64_t ldw, const double* U, int64_t ldu, double target_bits,
                         const wsic_wf_opts* opts, double* c_out, double* rate_out,
                         int32_t* passes_out, int32_t* codes, int64_t ldq, float* resid,
                         int64_t ldr, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    WSIC_TRY(check_layer(W, dtype, n_out, n_in, ldw));
    if (!U || ldu < n_in || !codes || ldq < n_in || (resid && ldr < n_in) || !c_out ||
        !rate_out || !(target_bits > 0.0) || !std::isfinite(target_bits)) {
      set_error("waterfill: bad argument");
      return WSIC_E_INVAL;
    }
    wsic_wf_opts o{WSIC_WF_RATE_TOL, std::ldexp(1.0, -20), 64, WSIC_WF_AUTO, 0.0, WSIC_RATE_POOLED, 0};
    if (opts) {
      o = *opts;
      if (!(o.rate_tol >= 0.0)) o.rate_tol = WSIC_WF_RATE_TOL;
      if (!(o.bracket_log2 > 0.0)) o.bracket_log2 = std::ldexp(1.0, -20);
      if (o.max_passes <= 0) o.max_passes = 64;
      if (o.mode != WSIC_WF_AUTO && o.mode != WSIC_WF_SECANT && o.mode != WSIC_WF_BISECT) {
        set_error("waterfill: unknown mode %d", o.mode);
        return WSIC_E_INVAL;
      }
      if (o.rate_mode != WSIC_RATE_POOLED && o.rate_mode != WSIC_RATE_COLUMNS) {
        set_error("waterfill: unknown rate mode %d", o.rate_mode);
        return WSIC_E_INVAL;
      }
    }
    if (o.mode == WSIC_WF_AUTO)
      o.mode = (n_out * n_in < WSIC_WF_AUTO_PARAMS) ? WSIC_WF_BISECT : WSIC_WF_SECANT;
    const bool cols = o.rate_mode == WSIC_RATE_COLUMNS;
    const bool trace = g_dbg.trace.load();
    WSIC_TRY(check_ws(lam ? WSIC_OP_SOFTWATER : WSIC_OP_WATERFILL, n_out, n_in, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    WfWs wf = carve_wf(cv, n_out, n_in);
    SicCtx x = make_ctx(n_out, n_in, W, dtype, ldw, U, ldu, wf.sic, st);
    if (lam) {
      const ScaleWs sc = carve_scales(cv, n_out);
      WSIC_TRY(launch_fill_zero(sc.flags, FLAGS_BYTES, st));
      WSIC_TRY(launch_row_sqrt(lam, n_out, sc.s, sc.flags, st));
      int sf = 0;
      WSIC_TRY(read_flags(sc.flags, &sf, st));
      WSIC_TRY(flags_status(sf, "softwater_waterfill"));
      x.rs = sc.s;
    }

    const double R = target_bits;
    // Starting grid scale: column variances of W and U's diagonal are read back while the setup
    // (Y = W U^T) runs; the setup's flags are read after it.
    double c0 = o.c_init;
    std::vector<double> gq;  // quantiles of std(W_:,j) U_jj for the secant's rate model
    int setup_flags = 0;
    if (!(c0 > 0.0)) {
      WSIC_TRY(launch_colstats(W, dtype, n_out, n_in, ldw, wf.colvar + (n_in + 1) / 2 * 2, wf.colvar,
                               st, x.rs));
      WSIC_TRY(launch_delta(U, ldu, n_in, 1.0, nullptr, wf.diag, st));
      std::vector<double> var(n_in), diag(n_in);
      const ReadPiece pv[2] = {{var.data(), wf.colvar, n_in * sizeof(double)},
                               {diag.data(), wf.diag, n_in * sizeof(double)}};
      WSIC_TRY(read_back_start(pv, 2, st));
      WSIC_TRY(sic_setup(x, false));
      WSIC_TRY(read_back_finish(pv, 2));
      double m = 0.0;
      for (int64_t j = 0; j < n_in; ++j) m += var[j] * diag[j] * diag[j];
      m /= (double)n_in;
      if (!(m > 0.0)) m = 1.0;
      // the oracle's high-rate start (the bisection replays the oracle's sequence from it)
      c0 = std::sqrt(2.0 * M_PI * M_E * m) * std::pow(2.0, -R);
      if (o.mode == WSIC_WF_SECANT && std::isfinite(c0)) {
        gq = scale_quantiles(var, diag);
        const double xm = model_solve(gq, R - 0.5 * o.rate_tol, std::log2(c0), !cols);
        if (std::isfinite(xm)) c0 = std::exp2(xm);
      }
    } else {
      WSIC_TRY(sic_setup(x, false));
    }
    WSIC_TRY(read_flags(x.ws.flags, &setup_flags, st));
    WSIC_TRY(flags_status(setup_flags, "sic"));

    // two code buffers: the caller's and one in the workspace; `hi_buf` holds the codes of
    // the best grid scale so far with H <= R
    // (the workspace pair is dense, row stride n_in; the caller's rows may be padded)
    int32_t* cbuf[2] = {codes, wf.codes2};
    float* rbuf[2] = {resid, resid ? wf.resid2 : nullptr};
    const int64_t qld[2] = {ldq, n_in};
    const int64_t rld[2] = {ldr, n_in};
    int passes = 0;
    int hi_buf = -1;
    double c_hi = 0, h_hi = 0, c_lo = 0, h_lo = 0;
    bool have_hi = false, have_lo = false;

    auto eval = [&](double c, int buf, double* H) -> int {
      if (passes >= o.max_passes) {
        set_error("waterfill: pass limit %d reached", o.max_passes);
        return WSIC_E_NO_BRACKET;
      }
      ++passes;
      WSIC_TRY(sic_pass_once(x, c, cbuf[buf], qld[buf], rbuf[buf], rld[buf]));
      int f = 0, nfix = 0, nchk = 0;
      auto rate_of = [&](int* fl, int* a1, int* a2) -> int {
        if (cols)
          return entropy_cols_of(cbuf[buf], n_out, n_in, qld[buf], wf.col, x.ws.pflags, st, H, fl,
                                 a1, a2);
        return entropy_of(cbuf[buf], n_out, n_in, qld[buf], wf.hist, x.ws.pflags, st, H, nullptr,
                          fl, a1, a2);
      };
      WSIC_TRY(rate_of(&f, &nfix, &nchk));
      if (x.i8 && (f & FLAG_OVERFLOW_LIST)) {  // a row listed too many large codes: fp64 pass
        SicCtx y = x;
        y.i8 = false;
        WSIC_TRY(sic_pass_once(y, c, cbuf[buf], qld[buf], rbuf[buf], rld[buf]));
        WSIC_TRY(rate_of(&f, nullptr, nullptr));
      }
      if (trace)
        std::fprintf(stderr,
                     "wsic waterfill pass %d: c=%.17g H=%.17g (%d decisions re-checked, %d "
                     "workgroups re-derived)\n",
                     passes, c, *H, nchk, nfix);
      return flags_status(f, "waterfill");
    };
    auto free_buf = [&]() { return hi_buf == 0 ? 1 : 0; };
    // record an evaluation at c into buffer b
    auto take = [&](double c, double h, int b) {
      if (h <= R) {
        if (!have_hi || c < c_hi) {
          c_hi = c;
          h_hi = h;
          hi_buf = b;
          have_hi = true;
        }
      } else {
        if (!have_lo || c > c_lo) {
          c_lo = c;
          h_lo = h;
          have_lo = true;
        }
      }
    };

    int rc = WSIC_OK;
    if (o.mode == WSIC_WF_BISECT) {
      // doubling/halving bracket, then geometric bisection on the bracket
      double c = c0, h;
      int b = free_buf();
      WSIC_TRY(eval(c, b, &h));
      take(c, h, b);
      int n = 0;
      while (h > R) {
        if (++n > 64) {
          set_error("waterfill: no bracket (rate stays above target)");
          return WSIC_E_NO_BRACKET;
        }
        c *= 2.0;
        b = free_buf();
        WSIC_TRY(eval(c, b, &h));
        take(c, h, b);
      }
      c = c_hi / 2.0;
      b = free_buf();
      WSIC_TRY(eval(c, b, &h));
      take(c, h, b);
      n = 0;
      while (h <= R) {
        if (++n > 64) {
          set_error("waterfill: no bracket (rate stays below target)");
          return WSIC_E_NO_BRACKET;
        }
        c = c / 2.0;
        b = free_buf();
        WSIC_TRY(eval(c, b, &h));
        take(c, h, b);
      }
      while (std::log2(c_hi / c_lo) > o.bracket_log2) {
        const double m = std::sqrt(c_lo * c_hi);
        b = free_buf();
        WSIC_TRY(eval(m, b, &h));
        take(m, h, b);
      }
    } else {
      // Secant on x = log2 c toward H = R - tol/2, from a start where a Gaussian-mixture rate
      // model (gauss_mix_entropy) gives R. The pooled entropy is not smooth at fine scales (a
      // grid change that flips one rounding decision re-routes the interference of every
      // column left of it), so before R is bracketed the slope is taken only from pairs of
      // evaluations at least SLOPE_DX apart (the model's slope for the first step); each step
      // starts from the latest evaluation. Once both sides of R are known the step must land
      // strictly inside the bracket, else -- or when the bracket has not halved in two steps --
      // bisect.
      constexpr double SLOPE_DX = 1.0 / 1024;
      const double Rt = R - 0.5 * o.rate_tol;
      auto accept = [&]() { return have_hi && h_hi > R - o.rate_tol; };
      // Probe (pooled rate): one pass over PROBE_K copies of S evenly spaced rows, copy g at the
      // grid scale c0 2^off[g] (rows are independent, so each copy quantizes exactly as its rows
      // would in the whole layer at that scale). The PROBE_K rates measure H(log2 c) around the
      // model's start; the first full pass goes to their crossing of Rt, and their local slope
      // replaces the model's. The sample's rate differs from the layer's by a near-constant
      // offset (~1e-3 bit at 512 x 4096 codes), which the first full pass measures and the
      // slope then removes.
      double probe_slope = 0.0;  // 0: no probe
      const int S = probe_rows(n_out);
      // (only with room for at least one full pass after it)
      if (!cols && S > 0 && wf.Yp && g_dbg.probe.load() && passes + 2 <= o.max_passes) {
        static const double off[PROBE_K] = {-0.16, -0.08, -0.04, -0.015, 0.015, 0.04, 0.08, 0.16};
        const double x0 = std::log2(c0);
        ProbeFactors fac{};
        for (int g = 0; g < PROBE_K; ++g) fac.v[g] = std::exp2(-off[g]);  // Y / c_g = (Y fac) / c0
        ++passes;
        WSIC_TRY(launch_probe_rows(x.ws.Y, n_in, n_out, n_in, S, PROBE_K, fac, wf.Yp, n_in, st));
        SicCtx xp = x;  // the probe layer shares U's operands and the pass buffers (S K <= n_out)
        xp.n_out = (int64_t)PROBE_K * S;
        xp.ws.Y = wf.Yp;
        WSIC_TRY(sic_pass_once(xp, c0, wf.codes2, n_in, nullptr, 0));
        WSIC_TRY(launch_fill_zero(wf.pbins, PROBE_K * PROBE_BIN_STRIDE * sizeof(unsigned long long),
                                  st));
        for (int g = 0; g < PROBE_K; ++g) {
          unsigned long long* bins = wf.pbins + g * PROBE_BIN_STRIDE;
          unsigned int* novf = reinterpret_cast<unsigned int*>(bins + HIST_BINS);
          WSIC_TRY(launch_hist(wf.codes2 + (size_t)g * S * n_in, S, n_in, n_in, bins, wf.hist.ovf,
                               novf, st));
          WSIC_TRY(launch_entropy_reduce(bins, novf, g == 0 ? x.ws.pflags : nullptr, wf.pres + g,
                                         st));
        }
        EntropyResult pr[PROBE_K];
        const ReadPiece rp{pr, wf.pres, sizeof pr};
        WSIC_TRY(read_back(&rp, 1, st));
        // a row whose list of large codes overflowed, or codes beyond the histogram's window:
        // the probe is dropped (the full passes handle both exactly)
        bool ok = !(pr[0].flags & FLAG_OVERFLOW_LIST);
        if (ok) WSIC_TRY(flags_status(pr[0].flags, "waterfill"));
        double xg[PROBE_K], hg[PROBE_K];
        const double Np = (double)S * (double)n_in;
        for (int g = 0; g < PROBE_K; ++g) {
          ok = ok && pr[g].ovf_count == 0;
          xg[g] = x0 + off[g];
          hg[g] = std::log2(Np) - pr[g].sum_nlogn / Np;
        }
        // the crossing of Rt on the piecewise-linear H(x) through the probes (H falls with x);
        // outside the probed range the end segment is extended
        int k = -1;
        for (int g = 0; g + 1 < PROBE_K && k < 0; ++g)
          if (hg[g] >= Rt && hg[g + 1] <= Rt) k = g;
        if (k < 0) k = (hg[PROBE_K - 1] > Rt) ? PROBE_K - 2 : 0;
        const double sl = (hg[k + 1] - hg[k]) / (xg[k + 1] - xg[k]);
        if (ok && sl < -0.25 && sl > -4.0) {
          const double x1 = std::min(x0 + 2.0, std::max(x0 - 2.0, xg[k] + (Rt - hg[k]) / sl));
          if (std::isfinite(x1)) {
            c0 = std::exp2(x1);
            probe_slope = sl;
          }
        }
        if (trace)
          std::fprintf(stderr,
                       "wsic waterfill pass %d: probe of %d scales on %d rows, H(c0 2^%.3f) = "
                       "%.6f ... H(c0 2^%.3f) = %.6f, slope %.5f, next c=%.17g%s\n",
                       passes, PROBE_K, S, off[0], hg[0], off[PROBE_K - 1], hg[PROBE_K - 1], sl,
                       c0, probe_slope != 0.0 ? "" : " (probe not used)");
      }
      std::vector<double> xs, hs;
      double xb = std::log2(c0), hb = 0.0;
      int b = free_buf();
      WSIC_TRY(eval(c0, b, &hb));
      take(c0, hb, b);
      xs.push_back(xb);
      hs.push_back(hb);
      double width_prev = INFINITY;
      int slow = 0;
      while (!accept()) {
        const bool bracketed = have_hi && have_lo;
        double xl = 0.0, xh = 0.0;
        if (bracketed) {
          xl = std::log2(c_lo);
          xh = std::log2(c_hi);
          if (xh - xl <= o.bracket_log2) break;
        }
        double slope = probe_slope != 0.0 ? probe_slope : -1.0;
        if (xs.size() == 1 && !gq.empty() && probe_slope == 0.0) {  // the rate model's slope
          const double dx = std::min(2.0, std::max(-2.0, hb - Rt));  // the step at slope -1
          if (std::fabs(dx) > 1e-9) {
            const double sl = (gauss_mix_entropy(gq, std::exp2(xb + dx), !cols) -
                               gauss_mix_entropy(gq, std::exp2(xb), !cols)) / dx;
            if (sl < -0.25 && sl > -4.0) slope = sl;
          }
        }
        // the latest evaluation far enough back (after a probe, whose slope rests on far more
        // codes than two nearby full passes resolve, only one much farther back)
        const double min_dx = probe_slope != 0.0 ? 1.0 / 64 : SLOPE_DX;
        for (size_t i = xs.size() - 1; i-- > 0;) {
          if (std::fabs(xb - xs[i]) >= min_dx) {
            const double sl = (hb - hs[i]) / (xb - xs[i]);
            if (sl < -0.25 && sl > -4.0) slope = sl;
            break;
          }
        }
        double xn = xb + (Rt - hb) / slope;
        if (bracketed) {
          // (interpolating between the bracket's ends instead was tried: more passes over 20
          // targets, the ends' rates being as noisy as the slope they would give)
          if (!(xn > xl && xn < xh) || slow >= 2) {
            xn = 0.5 * (xl + xh);
            slow = 0;
          }
        } else {
          xn = std::min(xb + 4.0, std::max(xb - 4.0, xn));
          const double tiny = std::ldexp(1.0, -30);
          if (!have_lo) xn = std::min(xn, xb - tiny);  // every H so far <= R: shrink c
          if (!have_hi) xn = std::max(xn, xb + tiny);  // every H so far > R: grow c
        }
        const double cn = std::exp2(xn);
        b = free_buf();
        double hn;
        WSIC_TRY(eval(cn, b, &hn));
        take(cn, hn, b);
        xb = xn;
        hb = hn;
        xs.push_back(xb);
        hs.push_back(hb);
        if (have_hi && have_lo) {
          const double width = std::log2(c_hi) - std::log2(c_lo);
          slow = (width > 0.5 * width_prev) ? slow + 1 : 0;
          width_prev = width;
        }
      }
      if (!have_hi) {
        set_error("waterfill: target not reached");
        return WSIC_E_NO_BRACKET;
      }
    }
    // the accepted codes must end in the caller's buffers
    if (hi_buf == 1) {
      // (dense rows: one linear copy, which the runtime runs faster than a 2-D one)
      if (ldq == n_in)
        WSIC_HIP_TRY(hipMemcpyAsync(codes, wf.codes2, (size_t)n_out * n_in * sizeof(int32_t),
                                    hipMemcpyDeviceToDevice, st));
      else
        WSIC_HIP_TRY(hipMemcpy2DAsync(codes, ldq * sizeof(int32_t), wf.codes2,
                                      n_in * sizeof(int32_t), n_in * sizeof(int32_t), n_out,
                                      hipMemcpyDeviceToDevice, st));
      if (resid && ldr == n_in)
        WSIC_HIP_TRY(hipMemcpyAsync(resid, wf.resid2, (size_t)n_out * n_in * sizeof(float),
                                    hipMemcpyDeviceToDevice, st));
      else if (resid)
        WSIC_HIP_TRY(hipMemcpy2DAsync(resid, ldr * sizeof(float), wf.resid2, n_in * sizeof(float),
                                      n_in * sizeof(float), n_out, hipMemcpyDeviceToDevice, st));
      WSIC_HIP_TRY(hipStreamSynchronize(st));
    }
    *c_out = c_hi;
    *rate_out = h_hi;
    if (passes_out) *passes_out = passes;
    return rc;
  } catch (...) {
    set_error("waterfill: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_waterfill(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                   const double* U, int64_t ldu, double target_bits, const wsic_wf_opts* opts,
                   double* c_out, double* rate_out, int32_t* passes_out, int32_t* codes,
                   int64_t ldq, float* resid, int64_t ldr, void* ws, size_t ws_bytes,
                   void* stream) {
  return waterfill_run(nullptr, W, dtype, n_out, n_in, ldw, U, ldu, target_bits, opts, c_out,
                       rate_out, passes_out, codes, ldq, resid, ldr, ws, ws_bytes, stream);
}

int wsic_softwater_waterfill(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                             const double* U, int64_t ldu, const double* lambda,
                             double target_bits, const wsic_wf_opts* opts, double* c_out,
                             double* rate_out, int32_t* passes_out, int32_t* codes, int64_t ldq,
                             float* resid, int64_t ldr, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (!lambda) {
    set_error("softwater_waterfill: lambda is required");
    return WSIC_E_INVAL;
  }
  return waterfill_run(lambda, W, dtype, n_out, n_in, ldw, U, ldu, target_bits, opts, c_out,
                       rate_out, passes_out, codes, ldq, resid, ldr, ws, ws_bytes, stream);
}

int wsic_softmax_curvature(const void* X, int dtype, int64_t rows, int64_t n_in, int64_t ldx,
                           const void* W, int64_t n_classes, int64_t ldw, double smoothing,
                           double alpha, double beta, double* lambda, void* ws, size_t ws_bytes,
                           void* stream) {
  try {
    clear_error();
    if (!X || !W || !lambda || rows <= 0 || n_in <= 0 || n_classes <= 0 || ldx < n_in ||
        ldw < n_in || (dtype != WSIC_F32 && dtype != WSIC_BF16) || !(smoothing >= 0.0) ||
        !(smoothing <= 1.0) || !std::isfinite(alpha) || !std::isfinite(beta)) {
      set_error("softmax_curvature: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_CURVATURE, rows, n_classes, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    const CurvWs cw = carve_curv(cv, rows, n_classes);
    WSIC_TRY(launch_fill_zero(cw.flags, FLAGS_BYTES, st));
    WSIC_TRY(launch_check_finite(X, dtype, rows, n_in, ldx, cw.flags, st));
    WSIC_TRY(launch_check_finite(W, dtype, n_classes, n_in, ldw, cw.flags, st));
    int f = 0;
    WSIC_TRY(read_flags(cw.flags, &f, st));
    WSIC_TRY(flags_status(f, "softmax_curvature"));
    CurvArgs a{};
    a.X = X;
    a.W = W;
    a.dtype = dtype;
    a.rows = rows;
    a.n = n_in;
    a.ldx = ldx;
    a.K = n_classes;
    a.ldw = ldw;
    a.eps = smoothing;
    a.alpha = alpha;
    a.beta = beta;
    a.lam = lambda;
    a.flags = cw.flags;
    a.Lg = cw.Lg;
    a.ldl = cw.ldl;
    a.part = cw.part;
    a.rmax = cw.rmax;
    a.rinvz = cw.rinvz;
    a.cpart = cw.cpart;
    // diagnostic switch: the fp64 VALU logits for bf16 inputs too
    a.force_generic = g_dbg.logits_generic.load();
    WSIC_TRY(launch_softmax_curvature(a, st));
    WSIC_TRY(read_flags(cw.flags, &f, st));
    return flags_status(f, "softmax_curvature");
  } catch (...) {
    set_error("softmax_curvature: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_softwater_distortion(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                              const double* U, int64_t ldu, double c, const double* lambda,
                              const float* resid, int64_t ldr, double* D_out, void* W_hat,
                              int w_hat_dtype, int64_t ldh, void* ws, size_t ws_bytes,
                              void* stream) {
  try {
    clear_error();
    if (!codes || n_out <= 0 || n_in <= 0 || ldq < n_in || !U || ldu < n_in || !(c > 0.0) ||
        !std::isfinite(c) || !lambda || !resid || ldr < n_in || !D_out ||
        (W_hat && (ldh < n_in || (w_hat_dtype != WSIC_F32 && w_hat_dtype != WSIC_BF16)))) {
      set_error("softwater_distortion: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_SOFTWATER_DIST, n_out, n_in, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    DistWs d = carve_dist(cv, n_out, n_in);
    const ScaleWs sc = carve_scales(cv, n_out);
    WSIC_TRY(launch_fill_zero(d.flags, FLAGS_BYTES, st));
    WSIC_TRY(launch_prep(U, ldu, n_in, d.invd, d.flags, st));
    WSIC_TRY(launch_row_sqrt(lambda, n_out, sc.s, d.flags, st));
    if (W_hat)
      WSIC_TRY(launch_dequant(codes, n_out, n_in, ldq, d.invd, c, W_hat, w_hat_dtype, ldh, st, sc.s));
    // the residuals of the class-aware SIC are those of the rows s_r w_r: sum_j U_jj^2 sum_r r_rj^2
    // is sum_r lambda_r e_r Sigma e_r^T, twice the KL estimate
    const int64_t np = dist_resid_partials(n_out, n_in);
    WSIC_TRY(launch_dist_resid(resid, n_out, n_in, ldr, U, ldu, d.partial, (int)np, st));
    WSIC_TRY(launch_sum_partials(d.partial, np, d.out, st));
    int f = 0;
    double D2 = 0.0;
    const ReadPiece pd[2] = {{&D2, d.out, sizeof(double)}, {&f, d.flags, sizeof(int)}};
    WSIC_TRY(read_back(pd, 2, st));
    *D_out = 0.5 * D2;
    return flags_status(f, "softwater_distortion");
  } catch (...) {
    set_error("softwater_distortion: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_entropy_columns(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                         double* bits_per_param, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    if (!codes || !bits_per_param || n_out <= 0 || n_in <= 0 || ldq < n_in) {
      set_error("entropy_columns: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_ENTROPY_COLUMNS, n_out, n_in, ws, ws_bytes));
    Carve cv(ws);
    cv.take<int>(FLAGS_BYTES / sizeof(int));
    const ColHistWs h = carve_colhist(cv, n_in);
    return entropy_cols_of(codes, n_out, n_in, ldq, h, nullptr, (hipStream_t)stream, bits_per_param);
  } catch (...) {
    set_error("entropy_columns: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_gaussian_rate(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                       const double* U, int64_t ldu, double D, double* rate_out, double* var_out,
                       void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    WSIC_TRY(check_layer(W, dtype, n_out, n_in, ldw));
    if (!U || ldu < n_in || !(D > 0.0) || !std::isfinite(D) || !rate_out) {
      set_error("gaussian_rate: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_GAUSS_RATE, n_out, n_in, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    int* flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
    double* part = cv.take<double>(SUMSQ_BLOCKS + 2);
    double* logd = cv.take<double>((size_t)n_in);
    double* sums = part + SUMSQ_BLOCKS;  // [0] sum w^2, [1] sum log2 U_jj
    const int64_t total = n_out * n_in;
    const int nblk = (int)std::min<int64_t>(SUMSQ_BLOCKS, (total + 255) / 256);
    WSIC_TRY(launch_fill_zero(flags, FLAGS_BYTES, st));
    WSIC_TRY(launch_sumsq(W, dtype, n_out, n_in, ldw, part, nblk, st));
    WSIC_TRY(launch_sum_partials(part, nblk, sums, st));
    WSIC_TRY(launch_logdiag(U, ldu, n_in, logd, flags, st));
    WSIC_TRY(launch_sum_partials(logd, n_in, sums + 1, st));
    double r[2] = {0.0, 0.0};
    int f = 0;
    const ReadPiece pr[2] = {{r, sums, sizeof r}, {&f, flags, sizeof(int)}};
    WSIC_TRY(read_back(pr, 2, st));
    WSIC_TRY(flags_status(f, "gaussian_rate"));
    const double var = r[0] / (double)total;
    const double theta = D / (double)total;
    *rate_out = 0.5 * std::log2(var / theta) + r[1] / (double)n_in;
    if (var_out) *var_out = var;
    return WSIC_OK;
  } catch (...) {
    set_error("gaussian_rate: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_lmmse_scale(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                     const double* U, int64_t ldu, const float* resid, int64_t ldr, double* gamma,
                     double* D_before, double* D_after, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    WSIC_TRY(check_layer(W, dtype, n_out, n_in, ldw));
    if (!U || ldu < n_in || !resid || ldr < n_in || !gamma) {
      set_error("lmmse_scale: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_LMMSE, n_out, n_in, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    int* flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
    double* Y = cv.take<double>((size_t)n_out * n_in);
    double* rows = cv.take<double>(3 * (size_t)n_out + 2);
    double* dbefore = rows;
    double* dafter = rows + n_out;
    double* sums = rows + 3 * n_out;
    WSIC_TRY(launch_fill_zero(flags, FLAGS_BYTES, st));
    WSIC_TRY(launch_prep(U, ldu, n_in, rows + 2 * n_out, flags, st));  // U diagonal checks
    const double work = (double)n_out * (double)n_in * (double)(n_in + 1);
    WSIC_TRY(launch_gemm_y(dtype, n_out, n_in, n_in, W, ldw, U, ldu, Y, n_in, work, st));
    WSIC_TRY(launch_lmmse_rows(Y, n_in, resid, ldr, U, ldu, n_out, n_in, gamma, dbefore, dafter, st));
    WSIC_TRY(launch_sum_partials(dbefore, n_out, sums, st));
    WSIC_TRY(launch_sum_partials(dafter, n_out, sums + 1, st));
    double r[2] = {0.0, 0.0};
    int f = 0;
    const ReadPiece pr[2] = {{r, sums, sizeof r}, {&f, flags, sizeof(int)}};
    WSIC_TRY(read_back(pr, 2, st));
    if (D_before) *D_before = r[0];
    if (D_after) *D_after = r[1];
    return flags_status(f, "lmmse_scale");
  } catch (...) {
    set_error("lmmse_scale: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_live_features(const double* Sigma, int64_t n, int64_t lds, double tau, int32_t* idx,
                       int32_t* pos, int64_t* n_live, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    if (!Sigma || n <= 0 || lds < n || !idx || !pos || !n_live || !(tau >= 0.0) || !(tau < 1.0)) {
      set_error("live_features: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_LIVE, 0, n, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    int* flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
    long long* cnt = cv.take<long long>(1);
    WSIC_TRY(launch_fill_zero(flags, FLAGS_BYTES, st));
    WSIC_TRY(launch_live_scan(Sigma, n, lds, tau, idx, pos, cnt, flags, st));
    long long c = 0;
    int f = 0;
    const ReadPiece pr[2] = {{&c, cnt, sizeof c}, {&f, flags, sizeof(int)}};
    WSIC_TRY(read_back(pr, 2, st));
    *n_live = c;
    WSIC_TRY(flags_status(f, "live_features"));
    if (c == 0) {
      set_error("live_features: every input column is dead");
      return WSIC_E_INVAL;
    }
    return WSIC_OK;
  } catch (...) {
    set_error("live_features: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_gather_features(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                         const double* Sigma, int64_t lds, const int32_t* idx, int64_t n_live,
                         void* W_live, int64_t ldwl, double* Sigma_live, int64_t ldsl,
                         void* stream) {
  try {
    clear_error();
    WSIC_TRY(check_layer(W, dtype, n_out, n_in, ldw));
    if (!idx || n_live <= 0 || n_live > n_in || !W_live || ldwl < n_live ||
        (Sigma && (lds < n_in || !Sigma_live || ldsl < n_live))) {
      set_error("gather_features: bad argument");
      return WSIC_E_INVAL;
    }
    return launch_gather_features(W, dtype, n_out, ldw, Sigma, lds, idx, n_live, W_live, ldwl,
                                  Sigma_live, ldsl, (hipStream_t)stream);
  } catch (...) {
    set_error("gather_features: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_scatter_codes(const int32_t* codes_live, int64_t n_out, int64_t ldql, const int32_t* pos,
                       int64_t n_in, int32_t* codes, int64_t ldq, void* stream) {
  try {
    clear_error();
    if (!codes_live || n_out <= 0 || ldql <= 0 || !pos || n_in <= 0 || !codes || ldq < n_in) {
      set_error("scatter_codes: bad argument");
      return WSIC_E_INVAL;
    }
    return launch_scatter_codes(codes_live, ldql, pos, n_in, n_out, codes, ldq, (hipStream_t)stream);
  } catch (...) {
    set_error("scatter_codes: internal exception");
    return WSIC_E_INVAL;
  }
}

size_t wsic_rans_bound(int64_t n, int32_t lane_symbols) {
  if (n <= 0 || lane_symbols <= 0) return 0;
  const int64_t G = rans_groups(n, lane_symbols);
  return rans_layout(G, RANS_MAX_SYM, n, n).total;
}

int wsic_rans_encode(const int32_t* codes, int64_t n, int32_t lane_symbols, uint8_t* out,
                     size_t out_cap, size_t* out_bytes, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    if (!codes || n <= 0 || lane_symbols <= 0 || lane_symbols > 65536 || !out || !out_bytes ||
        n > 0x7fffffffLL) {
      set_error("rans_encode: bad argument");
      return WSIC_E_INVAL;
    }
    const int L = lane_symbols;
    const int64_t G = rans_groups(n, L);
    if (out_cap < wsic_rans_bound(n, L)) {
      set_error("rans_encode: output capacity %zu below the bound %zu", out_cap, wsic_rans_bound(n, L));
      return WSIC_E_WORKSPACE;
    }
    WSIC_TRY(check_ws(WSIC_OP_RANS_ENC, L, n, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    cv.take<int>(FLAGS_BYTES / sizeof(int));
    const HistWs h = carve_hist(cv);
    uint32_t* cnt = cv.take<uint32_t>(2 * (size_t)G + 2);
    uint32_t* gwords = cnt + G;
    uint16_t* temp = cv.take<uint16_t>((size_t)G * 64 * (size_t)L);
    // table from the pooled histogram (window +-2047; wider codes are the escapes)
    WSIC_TRY(launch_fill_zero(h.bins, HIST_CLEAR_BYTES, st));
    WSIC_TRY(launch_hist(codes, 1, n, n, h.bins, h.ovf, h.ovf_count, st));
    std::vector<unsigned long long> bins(HIST_BINS);
    unsigned novf = 0;
    const ReadPiece pb[2] = {{bins.data(), h.bins, HIST_BINS * sizeof(unsigned long long)},
                             {&novf, h.ovf_count, sizeof(unsigned)}};
    WSIC_TRY(read_back(pb, 2, st));
    int lo = 0, hi = 0;
    bool any = false;
    for (int b = 0; b < HIST_BINS; ++b)
      if (bins[b]) {
        if (!any) lo = b - HIST_HALF;
        hi = b - HIST_HALF;
        any = true;
      }
    const int nsym = hi - lo + 2;
    std::vector<int64_t> counts(nsym, 0);
    for (int v = lo; v <= hi && any; ++v) counts[v - lo] = (int64_t)bins[v + HIST_HALF];
    counts[nsym - 1] = (int64_t)novf;
    const std::vector<uint16_t> freq = rans_normalize(counts, n);
    // escape offsets, then the layout (payload size is known after encoding); the sections before
    // the escapes and the padding after them are cleared first, so the container is fully defined
    WSIC_TRY(launch_rans_esc_count(codes, n, L, G, cnt, st));
    RansLayout lay = rans_layout(G, nsym, 0, 0);
    WSIC_TRY(launch_fill_zero(out, lay.esc, st));
    uint32_t* eofs = (uint32_t*)(out + lay.eofs);
    WSIC_TRY(launch_scan_u32(cnt, G, eofs, st));
    // the histogram counted the escapes already; the scan's total is checked against it with the
    // payload's length below (the escapes written stay inside the container's bound either way)
    const uint32_t n_esc = novf;
    lay = rans_layout(G, nsym, n_esc, 0);
    if (lay.payload > lay.esc + 4 * (size_t)n_esc)
      WSIC_TRY(launch_fill_zero(out + lay.esc + 4 * (size_t)n_esc, lay.payload - lay.esc - 4 * (size_t)n_esc, st));
    WSIC_HIP_TRY(hipMemcpyAsync(out + lay.freq, freq.data(), 2 * freq.size(), hipMemcpyHostToDevice, st));
    WSIC_TRY(launch_rans_encode(codes, n, L, G, lo, nsym, (const uint16_t*)(out + lay.freq), eofs,
                                (int32_t*)(out + lay.esc), temp, gwords, (uint32_t*)(out + lay.states), st));
    uint32_t* gofs = (uint32_t*)(out + lay.gofs);
    WSIC_TRY(launch_scan_u32(gwords, G, gofs, st));
    uint32_t nw = 0, n_esc_scan = 0;
    const ReadPiece pw[2] = {{&nw, gofs + G, sizeof(uint32_t)},
                             {&n_esc_scan, eofs + G, sizeof(uint32_t)}};
    WSIC_TRY(read_back(pw, 2, st));
    if (n_esc_scan != n_esc) {
      set_error("rans_encode: internal: %u escapes counted, %u in the histogram", n_esc_scan, n_esc);
      return WSIC_E_INVAL;
    }
    lay = rans_layout(G, nsym, n_esc, nw);
    WSIC_TRY(launch_rans_compact(temp, L, G, gwords, gofs, (uint16_t*)(out + lay.payload), st));
    uint32_t hdr[16] = {RANS_MAGIC, 1u, (uint32_t)(n & 0xffffffffLL), (uint32_t)(n >> 32), (uint32_t)L,
                        (uint32_t)G, (uint32_t)lo, (uint32_t)nsym, RANS_PROB, n_esc, nw, 0, 0, 0, 0, 0};
    WSIC_HIP_TRY(hipMemcpyAsync(out, hdr, sizeof hdr, hipMemcpyHostToDevice, st));
    WSIC_HIP_TRY(hipStreamSynchronize(st));  // the host buffers of the copies above
    *out_bytes = lay.total;
    return WSIC_OK;
  } catch (...) {
    set_error("rans_encode: internal exception");
    return WSIC_E_INVAL;
  }
}

// clear_flags false: the caller cleared the flags and queued kernels that may set them (their
// verdict is read back with the decode's)
static int rans_decode_any(const uint8_t* in, size_t in_bytes, int mode, void* dst, int64_t n,
                           int64_t n_in, const double* invd, double c, int* flags, hipStream_t st,
                           bool clear_flags = true) {
  if (in_bytes < 64) {
    set_error("rans_decode: container too short");
    return WSIC_E_INVAL;
  }
  uint32_t hdr[16];
  WSIC_HIP_TRY(hipMemcpyAsync(hdr, in, sizeof hdr, hipMemcpyDeviceToHost, st));
  WSIC_HIP_TRY(hipStreamSynchronize(st));
  const int64_t N = (int64_t)hdr[2] | ((int64_t)hdr[3] << 32);
  const int L = (int)hdr[4];
  const int64_t G = hdr[5];
  const int lo = (int)hdr[6];
  const int nsym = (int)hdr[7];
  if (hdr[0] != RANS_MAGIC || hdr[1] != 1u || hdr[8] != RANS_PROB || L <= 0 || nsym < 2 ||
      nsym > RANS_MAX_SYM || G != rans_groups(N, L)) {
    set_error("rans_decode: not a code container");
    return WSIC_E_INVAL;
  }
  if (N != n) {
    set_error("rans_decode: container holds %lld codes, %lld expected", (long long)N, (long long)n);
    return WSIC_E_INVAL;
  }
  const RansLayout lay = rans_layout(G, nsym, hdr[9], hdr[10]);
  if (in_bytes < lay.total) {
    set_error("rans_decode: container truncated (%zu of %zu bytes)", in_bytes, lay.total);
    return WSIC_E_INVAL;
  }
  if (clear_flags) WSIC_TRY(launch_fill_zero(flags, FLAGS_BYTES, st));
  WSIC_TRY(launch_rans_decode(mode, (const uint16_t*)(in + lay.freq), nsym, lo, N, L, G,
                              (const uint32_t*)(in + lay.gofs), (const uint32_t*)(in + lay.eofs),
                              (const uint32_t*)(in + lay.states), (const int32_t*)(in + lay.esc),
                              hdr[9], (const uint16_t*)(in + lay.payload), hdr[10], dst, n_in, invd, c,
                              flags, st));
  int f = 0;
  WSIC_TRY(read_flags(flags, &f, st));
  if (f & FLAG_RANGE) {
    set_error("rans_decode: corrupt container (a frequency table that does not sum to 2^14, a "
              "read past the escapes or the payload, or a stream that did not end in its start "
              "state)");
    return WSIC_E_INVAL;
  }
  return flags_status(f, "rans_decode");
}

int wsic_rans_decode(const uint8_t* in, size_t in_bytes, int32_t* codes, int64_t n, void* ws,
                     size_t ws_bytes, void* stream) {
  try {
    clear_error();
    if (!in || !codes || n <= 0) {
      set_error("rans_decode: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_RANS_DEC, 1, 1, ws, ws_bytes));
    return rans_decode_any(in, in_bytes, 0, codes, n, 1, nullptr, 0.0, (int*)ws, (hipStream_t)stream);
  } catch (...) {
    set_error("rans_decode: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_rans_decode_dequant(const uint8_t* in, size_t in_bytes, int64_t n_out, int64_t n_in,
                             const double* U, int64_t ldu, double c, void* W_hat, int w_hat_dtype,
                             void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    if (!in || n_out <= 0 || n_in <= 0 || !U || ldu < n_in || !(c > 0.0) || !std::isfinite(c) ||
        !W_hat || (w_hat_dtype != WSIC_F32 && w_hat_dtype != WSIC_BF16)) {
      set_error("rans_decode_dequant: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_RANS_DEC, 1, n_in, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    int* flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
    double* invd = cv.take<double>((size_t)n_in);
    // the column scales are formed while the container's header is read back; a bad diagonal
    // of U is reported with the decode's own verdict (the decode only multiplies by the scales)
    WSIC_TRY(launch_fill_zero(flags, FLAGS_BYTES, st));
    WSIC_TRY(launch_prep(U, ldu, n_in, invd, flags, st));
    return rans_decode_any(in, in_bytes, w_hat_dtype == WSIC_BF16 ? 2 : 1, W_hat, n_out * n_in, n_in,
                           invd, c, flags, st, false);
  } catch (...) {
    set_error("rans_decode_dequant: internal exception");
    return WSIC_E_INVAL;
  }
}

int wsic_entropy(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                 double* bits_per_param, int64_t* n_symbols, void* ws, size_t ws_bytes,
                 void* stream) {
  try {
    clear_error();
    if (!codes || !bits_per_param || n_out <= 0 || n_in <= 0 || ldq < n_in) {
      set_error("entropy: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_ENTROPY, n_out, n_in, ws, ws_bytes));
    Carve cv(ws);
    int* flags = cv.take<int>(FLAGS_BYTES / sizeof(int));
    HistWs h = carve_hist(cv);
    (void)flags;
    return entropy_of(codes, n_out, n_in, ldq, h, nullptr, (hipStream_t)stream, bits_per_param,
                      n_symbols, nullptr);
  } catch (...) {
    set_error("entropy: internal exception");
    return WSIC_E_INVAL;
  }
}

}  // extern "C"

namespace wsic {
namespace {
// Shared by wsic_distortion (caller's workspace, pinned staging for the read-back) and
// wsic_distortion_noalloc (the static scratch, a plain copy into the caller's host memory: no
// allocation of any kind).
int distortion_run(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                   const int32_t* codes, int64_t ldq, const double* U, int64_t ldu, double c,
                   const float* resid, int64_t ldr, int mode, double* D_out, void* W_hat,
                   int w_hat_dtype, int64_t ldh, void* ws, size_t ws_bytes, void* stream,
                   bool staged_readback) {
  try {
    WSIC_TRY(check_layer(W, dtype, n_out, n_in, ldw));
    if (!codes || ldq < n_in || !U || ldu < n_in || !(c > 0.0) || !std::isfinite(c) || !D_out ||
        (mode != WSIC_D_RESID && mode != WSIC_D_DIRECT) || (mode == WSIC_D_RESID && !resid) ||
        (resid && ldr < n_in) ||
        (W_hat && (ldh < n_in || (w_hat_dtype != WSIC_F32 && w_hat_dtype != WSIC_BF16)))) {
      set_error("distortion: bad argument");
      return WSIC_E_INVAL;
    }
    WSIC_TRY(check_ws(WSIC_OP_DISTORTION, n_out, n_in, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    Carve cv(ws);
    DistWs d = carve_dist(cv, n_out, n_in);
    WSIC_TRY(launch_fill_zero(d.flags, FLAGS_BYTES, st));
    WSIC_TRY(launch_prep(U, ldu, n_in, d.invd, d.flags, st));
    if (W_hat)
      WSIC_TRY(launch_dequant(codes, n_out, n_in, ldq, d.invd, c, W_hat, w_hat_dtype, ldh, st));
    int64_t np = 0;
    if (mode == WSIC_D_RESID) {
      np = dist_resid_partials(n_out, n_in);
      WSIC_TRY(launch_dist_resid(resid, n_out, n_in, ldr, U, ldu, d.partial, (int)np, st));
    } else {
      WSIC_TRY(launch_delta(U, ldu, n_in, c, d.delta, nullptr, st));
      GemmArgs g{};
      g.M = n_out;
      g.N = n_in;
      g.K = n_in;
      g.A = W;
      g.lda = ldw;
      g.Q = codes;
      g.ldq = ldq;
      g.vec = d.delta;
      g.B = U;
      g.ldb = ldu;
      g.alpha = 1.0;
      g.tri = 1;
      g.partial = d.partial;
      np = gemm_tiles(g);
      const double work = (double)n_out * (double)n_in * (double)(n_in + 1);
      WSIC_TRY(launch_gemm(dtype == WSIC_BF16 ? A_ERR_BF16 : A_ERR_F32, EPI_SUMSQ, g, "gemm_dist",
                           work, st));
    }
    WSIC_TRY(launch_sum_partials(d.partial, np, d.out, st));
    int f = 0;
    if (staged_readback) {
      const ReadPiece pd[2] = {{D_out, d.out, sizeof(double)}, {&f, d.flags, sizeof(int)}};
      WSIC_TRY(read_back(pd, 2, st));
    } else {
      double dh = 0.0;
      WSIC_HIP_TRY(hipMemcpyAsync(&dh, d.out, sizeof(double), hipMemcpyDeviceToHost, st));
      WSIC_HIP_TRY(hipMemcpyAsync(&f, d.flags, sizeof(int), hipMemcpyDeviceToHost, st));
      WSIC_HIP_TRY(hipStreamSynchronize(st));
      *D_out = dh;
    }
    return flags_status(f, "distortion");
  } catch (...) {
    set_error("distortion: internal exception");
    return WSIC_E_INVAL;
  }
}
}  // namespace
}  // namespace wsic

extern "C" {

int wsic_distortion(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                    const int32_t* codes, int64_t ldq, const double* U, int64_t ldu, double c,
                    const float* resid, int64_t ldr, int mode, double* D_out, void* W_hat,
                    int w_hat_dtype, int64_t ldh, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  return distortion_run(W, dtype, n_out, n_in, ldw, codes, ldq, U, ldu, c, resid, ldr, mode, D_out,
                        W_hat, w_hat_dtype, ldh, ws, ws_bytes, stream, true);
}

int wsic_distortion_noalloc(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                            const int32_t* codes, int64_t ldq, const double* U, int64_t ldu,
                            double c, const float* resid, int64_t ldr, int mode, double* D_out,
                            void* W_hat, int w_hat_dtype, int64_t ldh, void* stream) {
  clear_error();
  if (n_out <= 0 || n_in <= 0) {
    set_error("distortion_noalloc: bad shape");
    return WSIC_E_INVAL;
  }
  const size_t need = ws_bytes_for(WSIC_OP_DISTORTION, n_out, n_in);
  if (need > WSIC_NOALLOC_SCRATCH_BYTES) {
    set_error("distortion_noalloc: a %lld x %lld layer needs %zu bytes of scratch, the static "
              "buffer holds %zu (use wsic_distortion with a workspace)",
              (long long)n_out, (long long)n_in, need, (size_t)WSIC_NOALLOC_SCRATCH_BYTES);
    return WSIC_E_WORKSPACE;
  }
  void* ws = nullptr;
  WSIC_TRY(scratch_ptr(&ws));
  return distortion_run(W, dtype, n_out, n_in, ldw, codes, ldq, U, ldu, c, resid, ldr, mode, D_out,
                        W_hat, w_hat_dtype, ldh, ws, WSIC_NOALLOC_SCRATCH_BYTES, stream, false);
}

int wsic_profile_enable(int on) {
  g_prof = on != 0;
  return WSIC_OK;
}

int wsic_profile_select(const char* families) {
  g_prof_only.clear();
  if (!families) return WSIC_OK;
  std::string cur;
  for (const char* p = families;; ++p) {
    if (*p == ',' || *p == 0) {
      if (!cur.empty()) g_prof_only.push_back(cur);
      cur.clear();
      if (*p == 0) break;
    } else {
      cur += *p;
    }
  }
  return WSIC_OK;
}

int wsic_profile_reset(void) {
  clear_error();
  WSIC_TRY(prof_collect());
  g_acc.clear();
  return WSIC_OK;
}

int wsic_profile_read(const char* name, int64_t* launches, double* total_ms, double* total_work) {
  clear_error();
  if (!name) {
    set_error("profile_read: null name");
    return WSIC_E_INVAL;
  }
  WSIC_TRY(prof_collect());
  auto it = g_acc.find(name);
  const ProfAcc a = (it == g_acc.end()) ? ProfAcc{} : it->second;
  if (launches) *launches = a.launches;
  if (total_ms) *total_ms = a.ms;
  if (total_work) *total_work = a.work;
  return WSIC_OK;
}

int wsic_profile_names(char* buf, size_t buf_bytes) {
  clear_error();
  WSIC_TRY(prof_collect());
  std::string s;
  for (auto& kv : g_acc) {
    if (!s.empty()) s += ",";
    s += kv.first;
  }
  if (!buf || buf_bytes == 0) return WSIC_E_INVAL;
  std::snprintf(buf, buf_bytes, "%s", s.c_str());
  return WSIC_OK;
}

}  // extern "C"
