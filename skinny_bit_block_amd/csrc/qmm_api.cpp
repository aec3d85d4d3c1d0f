// C ABI of the skinny quantized product: argument checks, the gfx950 launch
// table, the split-K workspace and the launch on the caller's stream.
//
// The launch table plays the role of the per-architecture switch tables of the
// pages ("sixi-asi 0.9", sections "What I got wrong in 0.8" and "The patch"):
// the row count at which the row-vector kernel hands over to the tiled kernel,
// and the launch shape (waves per workgroup, split-K) that keeps enough loads
// in flight. A wrong entry there cost the pages' 8-row pass 163 vs 88 ms.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/qmm.h"
#include "qmm_internal.h"

// Cached occupancy query: workgroups per compute unit for one launch shape.
struct qmm_occ {
  int kernel, M, waves, lds, wgs;
};

struct qmm_ctx {
  int device;           // -1: planning-only handle (no device, no workspace)
  int cus;              // compute units
  qmm_occ occ[64];      // small cache of occupancy queries (launch shapes seen)
  int nocc;
  int forced_kernel;    // QMM_KERNEL_*
  int force_waves, force_splits, force_grid, force_wsplit;
  float* ws;            // split-K partials
  int64_t ws_bytes;
  unsigned* counters;   // split-K arrival counters, one per row tile, zeroed at creation
  int64_t max_counter_tiles;  // row tiles the counters cover
  bool fixed_scratch;   // the static scratch: a plan that does not fit is QMM_ERR_SCRATCH
  hipEvent_t ev_start, ev_stop;  // events for the next launch only (measurement)
};

namespace {

constexpr int64_t kWorkspaceBytes = 128ll << 20;
constexpr int kGfx950Cus = 256;
constexpr int kDefaultWaves = 4;
// Split K until there are at least this many row tiles of work (a wave per
// tile); below that the chip cannot keep enough loads in flight.
constexpr int64_t kTargetTiles = 1024;
constexpr int kMinBlocksPerSlice = 4;

int check_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > QMM_MAX_M || N < 1 || N > (int64_t)INT32_MAX / 32 || K < 256 ||
      K % 256 != 0 || K > (int64_t)1 << 24)
    return QMM_ERR_SHAPE;
  return QMM_OK;
}

// Measured entries of the launch table (gfx950, MI355X): the fastest
// (kernel, waves per workgroup, K slices, slices per workgroup) of a sweep, timed
// on the distinct matrices of a model pass in sequence (cold weights), per
// matrix shape of the pass and per range of rows; rows between measured
// points take the entry below them.
struct TableEntry {
  int32_t N, K, m_lo, kernel, waves, splits, wsplit;
  int32_t fmt = 0;  // 0: 4.5-bit super-blocks; 1: block-scaled FP4 groups; 2: plain INT4
  int32_t one_tile = 0;  // 1: a workgroup per tile group (no residency cap; the
                         // dispatcher balances the tail)
};
constexpr TableEntry kTable[] = {
    // 5120 x 5120 projections
    {5120, 5120, 1, QMM_KERNEL_VECTOR, 4, 2, 2},
    {5120, 5120, 2, QMM_KERNEL_TILED, 4, 2, 2},
    {5120, 5120, 5, QMM_KERNEL_TILED, 4, 3, 1},
    // gate+up, N = 2 x 17408
    {34816, 5120, 1, QMM_KERNEL_VECTOR, 2, 2, 2},
    {34816, 5120, 2, QMM_KERNEL_TILED, 3, 1, 1},
    {34816, 5120, 5, QMM_KERNEL_TILED, 6, 2, 2},
    {34816, 5120, 9, QMM_KERNEL_TILED, 6, 2, 1},
    {34816, 5120, 17, QMM_KERNEL_TILED, 8, 4, 1},
    // down
    {5120, 17408, 1, QMM_KERNEL_VECTOR, 4, 6, 2},
    {5120, 17408, 2, QMM_KERNEL_TILED, 4, 6, 2},
    {5120, 17408, 4, QMM_KERNEL_TILED, 8, 6, 2},
    {5120, 17408, 5, QMM_KERNEL_TILED, 8, 6, 1},  // 5..8 rows stage 8 row slots of x
    {5120, 17408, 9, QMM_KERNEL_TILED, 4, 6, 1, 0, 1},  // 9..16: 16 slots
    {5120, 17408, 17, QMM_KERNEL_TILED, 6, 12, 1},
    // single 2048 x 2048 projection (4 rows): every slice in one workgroup
    {2048, 2048, 4, QMM_KERNEL_TILED, 4, 4, 4},
    // five same-input 5120-wide projections as one call (N = 5 x 5120)
    {25600, 5120, 1, QMM_KERNEL_VECTOR, 8, 1, 1},
    {25600, 5120, 2, QMM_KERNEL_TILED, 8, 1, 1},
    {25600, 5120, 9, QMM_KERNEL_TILED, 8, 2, 1},
    {25600, 5120, 17, QMM_KERNEL_TILED, 8, 4, 1},
    // lm_head
    {151936, 5120, 1, QMM_KERNEL_VECTOR, 8, 1, 1},
    {151936, 5120, 2, QMM_KERNEL_TILED, 8, 1, 1},
    {151936, 5120, 16, QMM_KERNEL_TILED, 8, 2, 1},
    // block-scaled FP4 gate+up (lighter dequantization: its own optimum)
    {34816, 5120, 1, QMM_KERNEL_TILED, 3, 1, 1, 1},
    {34816, 5120, 5, QMM_KERNEL_TILED, 6, 2, 2, 1},
    {34816, 5120, 9, QMM_KERNEL_TILED, 6, 2, 1, 1},
    // plain INT4 (always tiled, two MFMA chains per group); rows below an
    // entry's first use the 4.5-bit entries
    {5120, 5120, 1, QMM_KERNEL_TILED, 4, 2, 2, 2},
    {5120, 5120, 9, QMM_KERNEL_TILED, 4, 3, 1, 2},
    {34816, 5120, 5, QMM_KERNEL_TILED, 6, 2, 2, 2},
    {34816, 5120, 9, QMM_KERNEL_TILED, 6, 2, 1, 2},
    {5120, 17408, 5, QMM_KERNEL_TILED, 4, 3, 1, 2},
    {5120, 17408, 9, QMM_KERNEL_TILED, 4, 6, 1, 2},
    {5120, 17408, 17, QMM_KERNEL_TILED, 6, 12, 1, 2},
};

// The entry for (M, N, K) and weight format fmt (the 4.5-bit entries when
// the table has none for fmt), or nullptr when the shape is not in the table.
const TableEntry* table_entry(int64_t M, int64_t N, int64_t K, int fmt = 0) {
  const TableEntry* best = nullptr;
  for (int want : {fmt, 0}) {
    for (const TableEntry& e : kTable)
      if (e.fmt == want && e.N == N && e.K == K && e.m_lo <= M && (!best || e.m_lo > best->m_lo))
        best = &e;
    if (best) break;
  }
  return best;
}

// The row count from which the launch table uses the tiled kernel: for a
// shape in the table the first entry that does; elsewhere two rows (where the
// sweeps put the switch for most shapes).
int table_switch(int64_t N, int64_t K) {
  for (int m = 1; m <= QMM_MAX_M; ++m) {
    const TableEntry* e = table_entry(m, N, K);
    if (!e) return 2;
    if (e->kernel == QMM_KERNEL_TILED) return m;
  }
  return QMM_MAX_M + 1;
}

// Workgroups of one launch shape the whole device holds at once; 0 when
// unknown (planning-only handle, or the query failed).
int64_t resident(qmm_ctx* h, int kernel, int M, int waves, int lds) {
  if (h->device < 0) return 0;
  for (int i = 0; i < h->nocc; ++i) {
    const qmm_occ& o = h->occ[i];
    if (o.kernel == kernel && o.M == M && o.waves == waves && o.lds == lds)
      return (int64_t)o.wgs * h->cus;
  }
  int prev = 0, wgs = 0;
  if (hipGetDevice(&prev) != hipSuccess) return 0;
  const bool sw = prev != h->device;
  if (sw && hipSetDevice(h->device) != hipSuccess) return 0;
  const hipError_t e = qmm::resident_per_cu(kernel, M, waves, lds, &wgs);
  if (sw) (void)hipSetDevice(prev);
  if (e != hipSuccess || wgs < 1) {
    (void)hipGetLastError();
    return 0;
  }
  const int slot = h->nocc < 64 ? h->nocc++ : (int)((uint32_t)(kernel * 131 + M * 31 + waves * 7 + lds) % 64u);
  h->occ[slot] = qmm_occ{kernel, M, waves, lds, wgs};
  return (int64_t)wgs * h->cus;
}

// slots > 0: an expert-indexed call (tiled kernel only), whose grid holds up
// to `slots` independent row groups; 0 for a plain call.
// fmt: 0 for 4.5-bit super-blocks; 1 a block-scaled FP4 call, 2 a plain INT4
// call (the tiled kernel, each format its own instantiation).
int make_plan(qmm_ctx* h, int64_t M, int64_t N, int64_t K, qmm_plan* p, int slots = 0,
              int fmt = 0) {
  const bool groups_fmt = fmt != 0;  // both group formats run the tiled kernel
  int rc = check_shape(M, N, K);
  if (rc) return rc;
  const int nb = (int)(K / 256);
  const int64_t ntiles = (N + 15) / 16;
  const TableEntry* te = table_entry(M, N, K, fmt);
  int kernel = M >= table_switch(N, K) ? QMM_KERNEL_TILED : QMM_KERNEL_VECTOR;
  if (te) kernel = te->kernel;
  if (h->forced_kernel != QMM_KERNEL_AUTO) kernel = h->forced_kernel;
  if (slots > 0) {
    if (h->forced_kernel == QMM_KERNEL_VECTOR) return QMM_ERR_INVALID_ARG;
    kernel = QMM_KERNEL_TILED;
    te = nullptr;  // table entries are for plain calls
  }
  if (kernel == QMM_KERNEL_VECTOR && M > qmm::kMaxVectorRows) return QMM_ERR_INVALID_ARG;
  if (groups_fmt) {
    if (h->forced_kernel == QMM_KERNEL_VECTOR) return QMM_ERR_INVALID_ARG;
    kernel = QMM_KERNEL_TILED;  // launch shape from the table: the same group geometry
  }
  const int groups_in_grid = slots > 0 ? slots : 1;
  // the instantiation that runs (its LDS and residency)
  const int kid = fmt == 1 ? 4 : (fmt == 2 ? 5 : (slots > 0 ? 3 : kernel));

  // without a table entry: 8 waves from 4096 row tiles of work in the grid
  // (an expert-indexed call streams one matrix per slot)
  const int waves = h->force_waves ? h->force_waves
                                   : (te ? te->waves
                                         : (ntiles * groups_in_grid >= 4096 ? 8 : kDefaultWaves));
  if (waves < 1 || waves > qmm::kMaxWavesPerWg) return QMM_ERR_INVALID_ARG;
  int wsplit = h->force_wsplit ? h->force_wsplit : (te ? te->wsplit : 1);
  // a table split that does not fit forced waves or slices falls back to 1
  if (!h->force_wsplit && (waves % wsplit || (h->force_splits && h->force_splits < wsplit)))
    wsplit = 1;
  if (wsplit < 1 || waves % wsplit) return QMM_ERR_INVALID_ARG;

  // K slices: the table's count, or enough tile-slices to fill the chip while
  // keeping at least a stage of super-blocks per slice; then raised until the
  // workgroup's staged x (wsplit slices) fits in LDS.
  int splits;
  if (h->force_splits) {
    splits = h->force_splits;
    if (splits < 1 || splits > nb) return QMM_ERR_INVALID_ARG;
  } else {
    int s_par = 1;
    if (te) {
      s_par = te->splits < nb ? te->splits : nb;
    } else {
      while (ntiles * s_par < kTargetTiles && (nb + s_par) / (s_par + 1) >= kMinBlocksPerSlice &&
             ntiles <= h->max_counter_tiles)
        ++s_par;
    }
    splits = s_par < wsplit ? wsplit : s_par;
    while (splits < nb &&
           qmm::lds_bytes((int)M, wsplit * ((nb + splits - 1) / splits), waves, wsplit, kid) >
               qmm::kLdsMax)
      ++splits;
  }
  if (splits < wsplit) return QMM_ERR_INVALID_ARG;
  const int nbs = (nb + splits - 1) / splits;
  splits = (nb + nbs - 1) / nbs;  // no empty slice
  const int grid_y = (splits + wsplit - 1) / wsplit;
  const int lds = qmm::lds_bytes((int)M, wsplit * nbs, waves, wsplit, kid);
  if (lds > qmm::kLdsMax) return QMM_ERR_INVALID_ARG;
  const int64_t ws = grid_y > 1 ? (int64_t)grid_y * M * N * 4 : 0;
  const int too_big = h->fixed_scratch ? QMM_ERR_SCRATCH : QMM_ERR_INVALID_ARG;
  if (ws > h->ws_bytes) return too_big;
  if (grid_y > 1 && ntiles * groups_in_grid > h->max_counter_tiles) return too_big;

  // at most one row tile per tile group of wsplit waves, and no more
  // workgroups than the device holds at once: the waves then walk several
  // tiles each (persistent grid)
  const int groups = waves / wsplit;
  const int64_t need = (ntiles + groups - 1) / groups;
  int64_t grid = need;
  const int64_t res = (te && te->one_tile) ? 0 : resident(h, kid, (int)M, waves, lds);
  if (res > 0) {
    const int64_t per_range =
        res / ((int64_t)grid_y * groups_in_grid) > 0 ? res / ((int64_t)grid_y * groups_in_grid) : 1;
    if (per_range < grid) grid = per_range;
  }
  if (h->force_grid) grid = h->force_grid;
  if (grid > 0x7FFFFFFF) return QMM_ERR_INVALID_ARG;

  p->kernel = kernel;
  p->waves_per_wg = waves;
  p->splits = splits;
  p->grid_x = (int32_t)grid;
  p->blocks_per_split = nbs;
  p->lds_bytes = lds;
  p->wave_splits = wsplit;
  p->workspace_bytes = ws;
  return QMM_OK;
}

// Measurement events set with qmm_set_launch_events go to the next launch only.
void take_events(qmm_ctx* h, qmm::Launch& a) {
  a.ev_start = h->ev_start;
  a.ev_stop = h->ev_stop;
  h->ev_start = h->ev_stop = nullptr;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

}  // namespace

extern "C" {

const char* qmm_status_string(int status) {
  switch (status) {
    case QMM_OK: return "QMM_OK";
    case QMM_ERR_INVALID_ARG: return "QMM_ERR_INVALID_ARG: null pointer or handle, or an override that does not fit the call";
    case QMM_ERR_SHAPE: return "QMM_ERR_SHAPE: need 1 <= M <= 32, N >= 1, K >= 256 and K % 256 == 0";
    case QMM_ERR_ALIGN: return "QMM_ERR_ALIGN: x and W_blocks must be 16-byte aligned, y 4-byte aligned";
    case QMM_ERR_NO_DEVICE: return "QMM_ERR_NO_DEVICE: no usable gfx950 device";
    case QMM_ERR_OOM: return "QMM_ERR_OOM: workspace allocation failed";
    case QMM_ERR_HIP: return "QMM_ERR_HIP: a HIP runtime call or kernel launch failed";
    case QMM_ERR_OVERLAP: return "QMM_ERR_OVERLAP: y overlaps x or W_blocks";
    case QMM_ERR_SCRATCH: return "QMM_ERR_SCRATCH: the call's split-K plan needs more than the static scratch holds (32 MiB of partial sums, 65536 row tiles); use qmm_run";
    default: return "QMM: unknown status";
  }
}

uint64_t qmm_weight_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % 256 != 0) return 0;
  return (uint64_t)N * (uint64_t)(K / 256) * 144u;
}

int qmm_create(qmm_handle* out, int device) {
  if (!out) return QMM_ERR_INVALID_ARG;
  *out = nullptr;
  qmm_ctx* h = new (std::nothrow) qmm_ctx();
  if (!h) return QMM_ERR_OOM;
  h->device = device;
  h->cus = kGfx950Cus;
  h->forced_kernel = QMM_KERNEL_AUTO;
  h->ws = nullptr;
  h->ws_bytes = kWorkspaceBytes;
  h->counters = nullptr;
  h->max_counter_tiles = qmm::kMaxCounterTiles;
  h->fixed_scratch = false;
  h->ev_start = h->ev_stop = nullptr;
  h->nocc = 0;
  if (device == -1) {  // planning-only handle
    *out = h;
    return QMM_OK;
  }
  int count = 0;
  if (device < 0 || hipGetDeviceCount(&count) != hipSuccess || device >= count) {
    delete h;
    return QMM_ERR_NO_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess ||
      std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    delete h;
    return QMM_ERR_NO_DEVICE;
  }
  h->cus = prop.multiProcessorCount;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess) {
    delete h;
    return QMM_ERR_HIP;
  }
  const char* inject = std::getenv("QMM_TEST_FAIL_ALLOC");  // failure-injection hook for tests
  hipError_t e = hipSuccess;
  if (!(inject && inject[0] == '1')) e = hipMalloc(reinterpret_cast<void**>(&h->ws), (size_t)h->ws_bytes);
  if (inject && inject[0] == '1') h->ws = nullptr;
  if (e == hipSuccess && h->ws)
    e = hipMalloc(reinterpret_cast<void**>(&h->counters), qmm::kMaxCounterTiles * sizeof(unsigned));
  if (e != hipSuccess || !h->ws || !h->counters) {
    (void)hipGetLastError();
    if (h->ws) (void)hipFree(h->ws);
    (void)hipSetDevice(prev);
    delete h;
    return QMM_ERR_OOM;
  }
  // the counters start at zero; every split-K call leaves them at zero
  e = hipMemset(h->counters, 0, qmm::kMaxCounterTiles * sizeof(unsigned));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = qmm::prepare_kernels();
  (void)hipSetDevice(prev);
  if (e != hipSuccess) {
    (void)hipFree(h->ws);
    (void)hipFree(h->counters);
    delete h;
    return QMM_ERR_HIP;
  }
  *out = h;
  return QMM_OK;
}

int qmm_destroy(qmm_handle h) {
  if (!h) return QMM_OK;
  if (h->ws || h->counters) {
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(h->device);
    if (h->ws) (void)hipFree(h->ws);
    if (h->counters) (void)hipFree(h->counters);
    (void)hipSetDevice(prev);
  }
  delete h;
  return QMM_OK;
}

int qmm_query_plan(qmm_handle h, int64_t M, int64_t N, int64_t K, qmm_plan* out) {
  if (!h || !out) return QMM_ERR_INVALID_ARG;
  return make_plan(h, M, N, K, out);
}

int qmm_query_plan_format(qmm_handle h, int format, int expert_slots, int64_t M, int64_t N,
                          int64_t K, qmm_plan* out) {
  if (!h || !out || format < QMM_FORMAT_KQUANT || format > QMM_FORMAT_INT4 || expert_slots < 0 ||
      (expert_slots > 0 && (format != QMM_FORMAT_KQUANT || expert_slots > M)))
    return QMM_ERR_INVALID_ARG;
  return make_plan(h, M, N, K, out, expert_slots, format);
}

int qmm_set_kernel(qmm_handle h, int kernel) {
  if (!h || kernel < QMM_KERNEL_AUTO || kernel > QMM_KERNEL_TILED) return QMM_ERR_INVALID_ARG;
  h->forced_kernel = kernel;
  return QMM_OK;
}

int qmm_set_shape(qmm_handle h, int waves_per_wg, int splits, int grid_x) {
  if (!h || waves_per_wg < 0 || splits < 0 || grid_x < 0) return QMM_ERR_INVALID_ARG;
  h->force_waves = waves_per_wg;
  h->force_splits = splits;
  h->force_grid = grid_x;
  return QMM_OK;
}

int qmm_set_wave_splits(qmm_handle h, int wave_splits) {
  if (!h || wave_splits < 0 || wave_splits > qmm::kMaxWavesPerWg) return QMM_ERR_INVALID_ARG;
  h->force_wsplit = wave_splits;
  return QMM_OK;
}

int qmm_set_launch_events(qmm_handle h, hipEvent_t start, hipEvent_t stop) {
  if (!h) return QMM_ERR_INVALID_ARG;
  h->ev_start = start;
  h->ev_stop = stop;
  return QMM_OK;
}

int qmm_switch_point(qmm_handle h, int64_t N, int64_t K) {
  if (!h) return QMM_ERR_INVALID_ARG;
  return table_switch(N, K);
}

int qmm_run(qmm_handle h, const float* x, const void* W_blocks, float* y, int64_t M, int64_t N,
            int64_t K, hipStream_t stream) {
  if (!h || !x || !W_blocks || !y) return QMM_ERR_INVALID_ARG;
  int rc = check_shape(M, N, K);
  if (rc) return rc;
  if (((uintptr_t)x & 15) || ((uintptr_t)W_blocks & 15) || ((uintptr_t)y & 3))
    return QMM_ERR_ALIGN;
  const size_t ybytes = (size_t)(M * N * 4);
  if (overlaps(y, ybytes, x, (size_t)(M * K * 4)) ||
      overlaps(y, ybytes, W_blocks, (size_t)qmm_weight_bytes(N, K)))
    return QMM_ERR_OVERLAP;
  qmm_plan p;
  rc = make_plan(h, M, N, K, &p);
  if (rc) return rc;
  if (h->device < 0) return QMM_ERR_NO_DEVICE;

  qmm::Launch a;
  a.kernel = p.kernel;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.waves_per_wg = p.waves_per_wg;
  a.wsplit = p.wave_splits;
  a.grid_x = p.grid_x;
  a.grid_y = (p.splits + p.wave_splits - 1) / p.wave_splits;
  a.nbs = p.blocks_per_split;
  a.xs_m = qmm::lds_xs_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.ss_m = qmm::lds_ss_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.lds_bytes = p.lds_bytes;
  a.x = x;
  a.W = W_blocks;
  a.y = y;
  a.ws = h->ws;
  a.counters = h->counters;
  a.ids = nullptr;
  a.E = 0;
  a.expert_bytes = 0;
  a.slots = 1;
  a.oscale = 1.0f;
  take_events(h, a);
  return qmm::launch(a, stream) == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}

int qmm_run_ids(qmm_handle h, const float* x, const void* W_experts, const int32_t* ids,
                int64_t E, float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (!h || !x || !W_experts || !ids || !y || E < 1) return QMM_ERR_INVALID_ARG;
  int rc = check_shape(M, N, K);
  if (rc) return rc;
  if (((uintptr_t)x & 15) || ((uintptr_t)W_experts & 15) || ((uintptr_t)y & 3) ||
      ((uintptr_t)ids & 3))
    return QMM_ERR_ALIGN;
  const uint64_t expert_bytes = qmm_weight_bytes(N, K);
  if ((uint64_t)E > (UINT64_MAX >> 1) / expert_bytes) return QMM_ERR_SHAPE;
  const size_t ybytes = (size_t)(M * N * 4);
  if (overlaps(y, ybytes, x, (size_t)(M * K * 4)) ||
      overlaps(y, ybytes, W_experts, (size_t)(expert_bytes * (uint64_t)E)) ||
      overlaps(y, ybytes, ids, (size_t)(M * 4)))
    return QMM_ERR_OVERLAP;
  const int slots = (int)(M < E ? M : E);
  qmm_plan p;
  rc = make_plan(h, M, N, K, &p, slots);
  if (rc) return rc;
  if (h->device < 0) return QMM_ERR_NO_DEVICE;
  qmm::Launch a;
  a.kernel = 3;  // the tiled kernel's expert-indexed instantiation
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.waves_per_wg = p.waves_per_wg;
  a.wsplit = p.wave_splits;
  a.grid_x = p.grid_x;
  a.grid_y = (p.splits + p.wave_splits - 1) / p.wave_splits;
  a.nbs = p.blocks_per_split;
  a.xs_m = qmm::lds_xs_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.ss_m = qmm::lds_ss_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.lds_bytes = p.lds_bytes;
  a.x = x;
  a.W = W_experts;
  a.y = y;
  a.ws = h->ws;
  a.counters = h->counters;
  a.ids = ids;
  a.E = (int)(E < 0x7FFFFFFF ? E : 0x7FFFFFFF);
  a.expert_bytes = (long long)expert_bytes;
  a.slots = slots;
  a.oscale = 1.0f;
  take_events(h, a);
  return qmm::launch(a, stream) == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}

int qmm_nvfp4_repack(const uint8_t* elems, const uint8_t* scales, int64_t N, int64_t K,
                     uint8_t* groups) {
  if (!elems || !scales || !groups) return QMM_ERR_INVALID_ARG;
  if (N < 1 || N > (int64_t)INT32_MAX / 32 || K < 256 || K % 256 != 0 || K > (int64_t)1 << 24)
    return QMM_ERR_SHAPE;
  const int64_t ng = K / 256;
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* er = elems + n * (K / 2);
    const uint8_t* sr = scales + n * (K / 16);
    for (int64_t b = 0; b < ng; ++b) {
      uint8_t* o = groups + (n * ng + b) * 144;
      std::memcpy(o, sr + b * 16, 16);  // scale codes of the group's 16 runs
      const uint8_t* eg = er + b * 128;  // the group's elements 0..255, two per byte
      for (int c = 0; c < 4; ++c)
        for (int r = 0; r < 32; ++r) {
          // element 64c + r to the low nibble, 64c + 32 + r to the high nibble
          const int lo = 64 * c + r, hi = lo + 32;
          const uint8_t qlo = (eg[lo >> 1] >> (4 * (lo & 1))) & 0xF;
          const uint8_t qhi = (eg[hi >> 1] >> (4 * (hi & 1))) & 0xF;
          o[16 + 32 * c + r] = (uint8_t)(qlo | (qhi << 4));
        }
    }
  }
  return QMM_OK;
}

int qmm_run_nvfp4(qmm_handle h, const float* x, const void* W_groups, float tensor_scale,
                  float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (!h || !x || !W_groups || !y || !std::isfinite(tensor_scale)) return QMM_ERR_INVALID_ARG;
  int rc = check_shape(M, N, K);
  if (rc) return rc;
  if (((uintptr_t)x & 15) || ((uintptr_t)W_groups & 15) || ((uintptr_t)y & 3))
    return QMM_ERR_ALIGN;
  const size_t ybytes = (size_t)(M * N * 4);
  if (overlaps(y, ybytes, x, (size_t)(M * K * 4)) ||
      overlaps(y, ybytes, W_groups, (size_t)qmm_weight_bytes(N, K)))
    return QMM_ERR_OVERLAP;
  qmm_plan p;
  rc = make_plan(h, M, N, K, &p, 0, 1);
  if (rc) return rc;
  if (h->device < 0) return QMM_ERR_NO_DEVICE;

  qmm::Launch a;
  a.kernel = 4;  // the tiled kernel's FP4 instantiation (its own x staging order)
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.waves_per_wg = p.waves_per_wg;
  a.wsplit = p.wave_splits;
  a.grid_x = p.grid_x;
  a.grid_y = (p.splits + p.wave_splits - 1) / p.wave_splits;
  a.nbs = p.blocks_per_split;
  a.xs_m = qmm::lds_xs_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.ss_m = qmm::lds_ss_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.lds_bytes = p.lds_bytes;
  a.x = x;
  a.W = W_groups;
  a.y = y;
  a.ws = h->ws;
  a.counters = h->counters;
  a.ids = nullptr;
  a.E = 0;
  a.expert_bytes = 0;
  a.slots = 1;
  a.oscale = tensor_scale;
  take_events(h, a);
  return qmm::launch(a, stream) == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}

int qmm_int4_repack(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                    uint8_t* groups) {
  if (!codes || !scales || !groups) return QMM_ERR_INVALID_ARG;
  if (N < 1 || N > (int64_t)INT32_MAX / 32 || K < 256 || K % 256 != 0 || K > (int64_t)1 << 24)
    return QMM_ERR_SHAPE;
  const int64_t ng = K / 256;
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* cr = codes + n * (K / 2);
    const uint16_t* sr = scales + n * (K / 128);
    for (int64_t b = 0; b < ng; ++b) {
      uint8_t* o = groups + (n * ng + b) * 144;
      std::memset(o, 0, 16);
      for (int j = 0; j < 2; ++j) {  // scales of elements 0..127 and 128..255, little-endian
        o[2 * j] = (uint8_t)(sr[2 * b + j] & 0xFF);
        o[2 * j + 1] = (uint8_t)(sr[2 * b + j] >> 8);
      }
      const uint8_t* cg = cr + b * 128;  // the group's elements 0..255, two per byte
      for (int c = 0; c < 4; ++c)
        for (int r = 0; r < 32; ++r) {
          // element 64c + r to the low nibble, 64c + 32 + r to the high nibble,
          // each code offset by 8 (two's complement q -> q + 8)
          const int lo = 64 * c + r, hi = lo + 32;
          const uint8_t qlo = ((cg[lo >> 1] >> (4 * (lo & 1))) & 0xF) ^ 0x8;
          const uint8_t qhi = ((cg[hi >> 1] >> (4 * (hi & 1))) & 0xF) ^ 0x8;
          o[16 + 32 * c + r] = (uint8_t)(qlo | (qhi << 4));
        }
    }
  }
  return QMM_OK;
}

int qmm_run_int4(qmm_handle h, const float* x, const void* W_groups, float* y, int64_t M,
                 int64_t N, int64_t K, hipStream_t stream) {
  if (!h || !x || !W_groups || !y) return QMM_ERR_INVALID_ARG;
  int rc = check_shape(M, N, K);
  if (rc) return rc;
  if (((uintptr_t)x & 15) || ((uintptr_t)W_groups & 15) || ((uintptr_t)y & 3))
    return QMM_ERR_ALIGN;
  const size_t ybytes = (size_t)(M * N * 4);
  if (overlaps(y, ybytes, x, (size_t)(M * K * 4)) ||
      overlaps(y, ybytes, W_groups, (size_t)qmm_weight_bytes(N, K)))
    return QMM_ERR_OVERLAP;
  qmm_plan p;
  rc = make_plan(h, M, N, K, &p, 0, 2);
  if (rc) return rc;
  if (h->device < 0) return QMM_ERR_NO_DEVICE;

  qmm::Launch a;
  a.kernel = 5;  // the tiled kernel's INT4 instantiation
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.waves_per_wg = p.waves_per_wg;
  a.wsplit = p.wave_splits;
  a.grid_x = p.grid_x;
  a.grid_y = (p.splits + p.wave_splits - 1) / p.wave_splits;
  a.nbs = p.blocks_per_split;
  a.xs_m = qmm::lds_xs_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.ss_m = qmm::lds_ss_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.lds_bytes = p.lds_bytes;
  a.x = x;
  a.W = W_groups;
  a.y = y;
  a.ws = h->ws;
  a.counters = h->counters;
  a.ids = nullptr;
  a.E = 0;
  a.expert_bytes = 0;
  a.slots = 1;
  a.oscale = 1.0f;
  take_events(h, a);
  return qmm::launch(a, stream) == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}

// The entry point that allocates nothing. Its context lives in a static
// table (one per device, set up at the first call on that device): the
// device's properties, the occupancy cache, and the static scratch of the
// kernel file as workspace.
namespace {
constexpr int kMaxStaticCtx = 64;
std::mutex g_static_mu;
qmm_ctx g_static_ctx[kMaxStaticCtx];
bool g_static_ready[kMaxStaticCtx];
}  // namespace

int qmm_run_static(const float* x, const void* W_blocks, float* y, int64_t M, int64_t N,
                   int64_t K, hipStream_t stream) {
  if (!x || !W_blocks || !y) return QMM_ERR_INVALID_ARG;
  int rc = check_shape(M, N, K);
  if (rc) return rc;
  if (((uintptr_t)x & 15) || ((uintptr_t)W_blocks & 15) || ((uintptr_t)y & 3))
    return QMM_ERR_ALIGN;
  const size_t ybytes = (size_t)(M * N * 4);
  if (overlaps(y, ybytes, x, (size_t)(M * K * 4)) ||
      overlaps(y, ybytes, W_blocks, (size_t)qmm_weight_bytes(N, K)))
    return QMM_ERR_OVERLAP;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxStaticCtx)
    return QMM_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_static_mu);
  qmm_ctx* h = &g_static_ctx[device];
  if (!g_static_ready[device]) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess ||
        std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return QMM_ERR_NO_DEVICE;
    void* scratch = nullptr;
    if (qmm::static_scratch(device, &scratch) != hipSuccess || qmm::prepare_kernels() != hipSuccess) {
      (void)hipGetLastError();
      return QMM_ERR_HIP;
    }
    h->device = device;
    h->cus = prop.multiProcessorCount;
    h->nocc = 0;
    h->forced_kernel = QMM_KERNEL_AUTO;
    h->force_waves = h->force_splits = h->force_grid = h->force_wsplit = 0;
    h->ws = static_cast<float*>(scratch);
    h->ws_bytes = (int64_t)qmm::kStaticPartialBytes;
    h->counters = reinterpret_cast<unsigned*>(static_cast<unsigned char*>(scratch) +
                                              qmm::kStaticPartialBytes);
    h->max_counter_tiles = qmm::kStaticCounterTiles;
    h->fixed_scratch = true;
    // the counters start at zero (and every split-K call leaves them so):
    // cleared once, on the caller's stream, ahead of the first launch
    if (qmm::clear_counters(h->counters, qmm::kStaticCounterTiles, stream) != hipSuccess)
      return QMM_ERR_HIP;
    g_static_ready[device] = true;
  }
  qmm_plan p;
  rc = make_plan(h, M, N, K, &p);
  if (rc) return rc;
  qmm::Launch a;
  a.kernel = p.kernel;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.waves_per_wg = p.waves_per_wg;
  a.wsplit = p.wave_splits;
  a.grid_x = p.grid_x;
  a.grid_y = (p.splits + p.wave_splits - 1) / p.wave_splits;
  a.nbs = p.blocks_per_split;
  a.xs_m = qmm::lds_xs_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.ss_m = qmm::lds_ss_m(p.wave_splits * p.blocks_per_split, p.kernel);
  a.lds_bytes = p.lds_bytes;
  a.x = x;
  a.W = W_blocks;
  a.y = y;
  a.ws = h->ws;
  a.counters = h->counters;
  a.ids = nullptr;
  a.E = 0;
  a.expert_bytes = 0;
  a.slots = 1;
  a.oscale = 1.0f;
  take_events(h, a);
  return qmm::launch(a, stream) == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}

}  // extern "C"
