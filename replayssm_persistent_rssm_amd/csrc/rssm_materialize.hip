// rssm_materialize.hip -- host side of librssm_materialize: validation of the
// host-visible arguments, instance selection, persistent-grid sizing and the
// launch on the caller's stream.  The C ABI is declared in rssm_materialize.h.
//
// Host validation mirrors the parameter rules of the flashinfer page for
// flashinfer.mamba.replayssm_materialize (heads_per_group divides num_heads;
// max_window in [1, 16]; one-byte state needs dim 64 and dstate 128; a seed
// when philox_rounds > 0) and the pull-request review's point that the head
// count must never be narrowed (here it is int32 by type, and the work size
// L*B*H is bounded so that the kernel's 64-bit item arithmetic cannot
// overflow).  Device metadata is never read on the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "gdn_kernel.h"
#include "rssm_gdn_commit.h"
#include "rssm_kernel.h"
#include "rssm_materialize.h"
#include "rssm_ssu_decode.h"
#include "ssu_kernel.h"

namespace rssm {
const KernelEntry* kernels_f32(int* n);
const KernelEntry* kernels_bf16(int* n);
const KernelEntry* kernels_f16(int* n);
const KernelEntry* kernels_i8(int* n);
const KernelEntry* kernels_f8(int* n);
const EncodeEntry* encoders_f32(int* n);
const EncodeEntry* encoders_bf16(int* n);
const EncodeEntry* encoders_f16(int* n);
const EncodeEntry* encoders_i8(int* n);
const EncodeEntry* encoders_f8(int* n);
const void* gdn_kernel_for(int window);
const void* ssu_kernel_for(int state_dtype, int input_dtype, int tokens);
}  // namespace rssm

namespace {

thread_local char g_err[1024];

rssm_status fail(rssm_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool verbose() {
  static const bool v = [] {
    const char* e = std::getenv("RSSM_MATERIALIZE_VERBOSE");
    return e != nullptr && *e != '\0' && std::strcmp(e, "0") != 0;
  }();
  return v;
}

const char* dtype_name(int d) {
  switch (d) {
    case RSSM_F32: return "f32";
    case RSSM_BF16: return "bf16";
    case RSSM_F16: return "f16";
    case RSSM_I8: return "i8";
    case RSSM_F8E4M3: return "f8e4m3";
    default: return "?";
  }
}

bool one_byte(int d) { return d == RSSM_I8 || d == RSSM_F8E4M3; }

template <typename T>
bool aligned(const T* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Compiled (dim, dstate) shapes.
bool shape_supported(int state_dtype, int dim, int dstate) {
  if (dim == 64 && dstate == 128) return true;
  return !one_byte(state_dtype) && dim == 16 && dstate == 16;
}

rssm_status validate_desc(const rssm_materialize_desc* d) {
  if (d == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->num_layers < 1) return fail(RSSM_ERR_INVALID_ARGUMENT, "num_layers must be >= 1 (got %d)", d->num_layers);
  if (d->batch < 1) return fail(RSSM_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", d->batch);
  if (d->num_heads < 1) return fail(RSSM_ERR_INVALID_ARGUMENT, "num_heads must be >= 1 (got %d)", d->num_heads);
  if (d->heads_per_group < 1 || d->num_heads % d->heads_per_group != 0)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "heads_per_group (%d) must be >= 1 and divide num_heads (%d)",
                d->heads_per_group, d->num_heads);
  if (d->dim < 1 || d->dstate < 1)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "dim and dstate must be >= 1 (got %d, %d)", d->dim, d->dstate);
  if (d->max_window < 1 || d->max_window > 16)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "max_window must be in [1, 16] (got %d)", d->max_window);
  if (d->ring_buffer_len < 1)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "ring_buffer_len must be >= 1 (got %d)", d->ring_buffer_len);
  if (d->philox_rounds < 0 || d->philox_rounds > 64)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "philox_rounds must be in [0, 64] (got %d)", d->philox_rounds);
  if (d->max_workgroups < 0)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "max_workgroups must be >= 0 (got %d)", d->max_workgroups);
  if (d->state_dtype < RSSM_F32 || d->state_dtype > RSSM_F8E4M3)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "unknown state_dtype %d", d->state_dtype);
  if (d->input_dtype < RSSM_F32 || d->input_dtype > RSSM_F8E4M3)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "unknown input_dtype %d", d->input_dtype);
  if (d->a_dtype < RSSM_F32 || d->a_dtype > RSSM_F8E4M3)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "unknown a_dtype %d", d->a_dtype);
  if (d->input_dtype != RSSM_F32 && d->input_dtype != RSSM_BF16 && d->input_dtype != RSSM_F16)
    return fail(RSSM_ERR_UNSUPPORTED, "input_dtype %s is not supported (f32, bf16, f16)", dtype_name(d->input_dtype));
  if (d->a_dtype != RSSM_F32)
    return fail(RSSM_ERR_UNSUPPORTED, "a_dtype %s is not supported (f32)", dtype_name(d->a_dtype));
  if (one_byte(d->state_dtype) && (d->dim != 64 || d->dstate != 128))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "one-byte state requires dim=64 and dstate=128 (got %d, %d)", d->dim,
                d->dstate);
  if (!shape_supported(d->state_dtype, d->dim, d->dstate))
    return fail(RSSM_ERR_UNSUPPORTED, "no compiled instance for dim=%d dstate=%d with %s state", d->dim, d->dstate,
                dtype_name(d->state_dtype));
  const int64_t work = static_cast<int64_t>(d->num_layers) * d->batch * d->num_heads;
  if (work > (int64_t(1) << 40))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "num_layers*batch*num_heads = %lld exceeds 2^40",
                static_cast<long long>(work));
  return RSSM_OK;
}

rssm_status validate_tables(const rssm_materialize_desc* d, const rssm_materialize_tables* t) {
  if (t == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "tables is NULL");
  struct P64 { const int64_t* p; const char* n; } p64[] = {
      {t->state_ptrs, "state_ptrs"}, {t->state_slot_strides, "state_slot_strides"},
      {t->x_ptrs, "x_ptrs"}, {t->x_slot_strides, "x_slot_strides"},
      {t->B_ptrs, "B_ptrs"}, {t->B_slot_strides, "B_slot_strides"},
      {t->dt_ptrs, "dt_ptrs"}, {t->dt_slot_strides, "dt_slot_strides"},
      {t->A_ptrs, "A_ptrs"}};
  for (const auto& e : p64) {
    if (e.p == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "%s is NULL", e.n);
    if (!aligned(e.p, 8)) return fail(RSSM_ERR_INVALID_ARGUMENT, "%s is not 8-byte aligned", e.n);
  }
  struct P32 { const int32_t* p; const char* n; } p32[] = {
      {t->src_slots, "src_slots"}, {t->dst_slots, "dst_slots"}, {t->ring_start, "ring_start"},
      {t->replay_prefix_len, "replay_prefix_len"}, {t->active_request_indices, "active_request_indices"}};
  for (const auto& e : p32) {
    if (e.p == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "%s is NULL", e.n);
    if (!aligned(e.p, 4)) return fail(RSSM_ERR_INVALID_ARGUMENT, "%s is not 4-byte aligned", e.n);
  }
  if (one_byte(d->state_dtype)) {
    if (t->scale_ptrs == nullptr || t->scale_slot_strides == nullptr)
      return fail(RSSM_ERR_INVALID_ARGUMENT, "one-byte state needs scale_ptrs and scale_slot_strides");
    if (!aligned(t->scale_ptrs, 8) || !aligned(t->scale_slot_strides, 8))
      return fail(RSSM_ERR_INVALID_ARGUMENT, "scale tables are not 8-byte aligned");
  }
  if (d->philox_rounds > 0) {
    if (t->rand_seed == nullptr)
      return fail(RSSM_ERR_INVALID_ARGUMENT, "rand_seed is required when philox_rounds > 0");
    if (!aligned(t->rand_seed, 8)) return fail(RSSM_ERR_INVALID_ARGUMENT, "rand_seed is not 8-byte aligned");
  }
  return RSSM_OK;
}

struct Registry {
  const rssm::KernelEntry* k[5];
  int nk[5];
  const rssm::EncodeEntry* e[5];
  int ne[5];
  Registry() {
    k[0] = rssm::kernels_f32(&nk[0]);
    k[1] = rssm::kernels_bf16(&nk[1]);
    k[2] = rssm::kernels_f16(&nk[2]);
    k[3] = rssm::kernels_i8(&nk[3]);
    k[4] = rssm::kernels_f8(&nk[4]);
    e[0] = rssm::encoders_f32(&ne[0]);
    e[1] = rssm::encoders_bf16(&ne[1]);
    e[2] = rssm::encoders_f16(&ne[2]);
    e[3] = rssm::encoders_i8(&ne[3]);
    e[4] = rssm::encoders_f8(&ne[4]);
  }
};

const Registry& registry() {
  static const Registry r;
  return r;
}

// nck: 1 for the single-checkpoint operation, rssm::kMaxCheckpoints for the
// multi-checkpoint instances.
const rssm::KernelEntry* find_kernel(const rssm_materialize_desc* d, int nck) {
  const int kmax = d->max_window <= 8 ? 8 : 16;
  const int sr = (d->philox_rounds > 0 && d->state_dtype != RSSM_F32) ? 1 : 0;
  const Registry& reg = registry();
  const int s = d->state_dtype;
  for (int i = 0; i < reg.nk[s]; ++i) {
    const rssm::KernelEntry& e = reg.k[s][i];
    if (e.it == d->input_dtype && e.dim == d->dim && e.dstate == d->dstate && e.kmax == kmax && e.sr == sr &&
        e.nck == nck)
      return &e;
  }
  return nullptr;
}

const rssm::EncodeEntry* find_encoder(const rssm_materialize_desc* d) {
  const int sr = (d->philox_rounds > 0 && d->state_dtype != RSSM_F32) ? 1 : 0;
  const Registry& reg = registry();
  const int s = d->state_dtype;
  for (int i = 0; i < reg.ne[s]; ++i) {
    const rssm::EncodeEntry& e = reg.e[s][i];
    if (e.dstate == d->dstate && e.sr == sr) return &e;
  }
  return nullptr;
}

// Cached device properties and per-kernel occupancy.
std::mutex g_mu;
std::unordered_map<int, int> g_cus;                      // device -> compute units
std::unordered_map<const void*, int> g_occ;              // kernel -> resident workgroups per CU

rssm_status grid_for(const void* fn, int* grid_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RSSM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_cus.find(dev);
  if (it == g_cus.end()) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(RSSM_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    it = g_cus.emplace(dev, cus).first;
  }
  auto ot = g_occ.find(fn);
  if (ot == g_occ.end()) {
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, rssm::kBlock, 0);
    if (e != hipSuccess) return fail(RSSM_ERR_HIP, "hipOccupancyMaxActiveBlocksPerMultiprocessor: %s",
                                     hipGetErrorString(e));
    ot = g_occ.emplace(fn, nb < 1 ? 1 : nb).first;
  }
  *grid_out = it->second * ot->second;
  return RSSM_OK;
}

// Default grid of the materialize kernels (the work loop is persistent either
// way).  A larger grid lets the hardware hand out workgroups as others
// finish, which balances requests of different cost; every workgroup also
// adds about 0.4 us per thousand to a call with nothing to do.  One-byte
// state with stochastic rounding (bound by VALU issue, per-request cost
// varying with the prefix length): eight times the resident capacity, which
// on MI355X ran the e4m3 + Philox-10 workload in 5.00 ms against 5.24 ms at
// four times and 5.86 ms at one (empty call 5.9 us against about 3.3 us).
// Other state, including one-byte state with nearest-even rounding: the
// resident capacity (int8 workload 2.30 ms at one, 2.29 ms at eight times).
rssm_status materialize_grid(const rssm_materialize_desc* d, const void* fn, int* grid_out) {
  int resident = 0;
  rssm_status st = grid_for(fn, &resident);
  if (st != RSSM_OK) return st;
  *grid_out = (one_byte(d->state_dtype) && d->philox_rounds > 0) ? 8 * resident : resident;
  return RSSM_OK;
}

// The last descriptor validated on this thread, with its instance and grid
// on that device: a serving loop calls with the same scalars every step.
struct LaunchCache {
  rssm_materialize_desc desc;
  int device = -1;
  int nck = 0;
  const rssm::KernelEntry* kernel = nullptr;
  int grid = 0;
};
thread_local LaunchCache g_last;

// Static LDS of a compiled kernel instance, in bytes (-1 if the query fails).
int lds_bytes_of(const void* fn) {
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, fn) != hipSuccess) return -1;
  return static_cast<int>(attr.sharedSizeBytes);
}

// Validate, pick the instance (cached per thread for an unchanged
// descriptor) and enqueue one launch.  ncp = 1 takes the single-checkpoint
// instances, ncp > 1 the multi-checkpoint ones.
rssm_status launch(const rssm_materialize_desc* desc, const rssm_materialize_tables* tables, int ncp,
                   void* hip_stream) {
  if (desc == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "desc is NULL");
  const int nck = ncp > 1 ? rssm::kMaxCheckpoints : 1;
  const rssm::KernelEntry* k = nullptr;
  int grid = 0;
  rssm_status st;
  const bool same_desc = g_last.kernel != nullptr && g_last.nck == nck &&
                         std::memcmp(&g_last.desc, desc, sizeof(rssm_materialize_desc)) == 0;
  // Host validation happens before any HIP call; an unchanged descriptor was
  // validated by an earlier call on this thread.
  if (!same_desc) {
    st = validate_desc(desc);
    if (st != RSSM_OK) return st;
  }
  st = validate_tables(desc, tables);
  if (st != RSSM_OK) return st;
  k = same_desc ? g_last.kernel : find_kernel(desc, nck);
  if (k == nullptr)
    return fail(RSSM_ERR_UNSUPPORTED, "no compiled %sinstance for state=%s input=%s dim=%d dstate=%d",
                nck > 1 ? "multi-checkpoint " : "", dtype_name(desc->state_dtype), dtype_name(desc->input_dtype),
                desc->dim, desc->dstate);
  int dev = 0;
  hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return fail(RSSM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(de));
  if (same_desc && g_last.device == dev) {
    grid = g_last.grid;
  } else {
    grid = desc->max_workgroups;
    if (grid == 0) {
      st = materialize_grid(desc, k->fn, &grid);
      if (st != RSSM_OK) return st;
    }
    g_last.desc = *desc;
    g_last.device = dev;
    g_last.nck = nck;
    g_last.kernel = k;
    g_last.grid = grid;
  }
  rssm::KernelArgs args;
  args.state_ptrs = tables->state_ptrs;
  args.state_strides = tables->state_slot_strides;
  args.x_ptrs = tables->x_ptrs;
  args.x_strides = tables->x_slot_strides;
  args.B_ptrs = tables->B_ptrs;
  args.B_strides = tables->B_slot_strides;
  args.dt_ptrs = tables->dt_ptrs;
  args.dt_strides = tables->dt_slot_strides;
  args.A_ptrs = tables->A_ptrs;
  args.scale_ptrs = tables->scale_ptrs;
  args.scale_strides = tables->scale_slot_strides;
  args.src_slots = tables->src_slots;
  args.dst_slots = tables->dst_slots;
  args.ring_start = tables->ring_start;
  args.prefix_len = tables->replay_prefix_len;
  args.active = tables->active_request_indices;
  args.rand_seed = tables->rand_seed;
  args.L = desc->num_layers;
  args.B = desc->batch;
  args.H = desc->num_heads;
  args.hpg = desc->heads_per_group;
  args.R = desc->ring_buffer_len;
  args.W = desc->max_window;
  args.pad = desc->pad_slot_id;
  args.rounds = desc->philox_rounds;
  args.ncp = ncp;
  if (verbose())
    std::fprintf(stderr, "[rssm_materialize] %s grid=%d block=%d lds=%dB L=%d B=%d H=%d checkpoints=%d\n", k->name,
                 grid, rssm::kBlock, lds_bytes_of(k->fn), desc->num_layers, desc->batch, desc->num_heads, ncp);
  void* params[] = {&args};
  hipError_t e = hipLaunchKernel(k->fn, dim3(grid), dim3(rssm::kBlock), params, 0,
                                 static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(RSSM_ERR_HIP, "launch of %s failed: %s", k->name, hipGetErrorString(e));
  return RSSM_OK;
}

}  // namespace

extern "C" {

const char* rssm_last_error(void) { return g_err; }

rssm_status rssm_materialize_launch_config(const rssm_materialize_desc* desc, int32_t* grid, int32_t* block,
                                           int32_t* lds_bytes) {
  g_err[0] = '\0';
  rssm_status st = validate_desc(desc);
  if (st != RSSM_OK) return st;
  if (grid == nullptr || block == nullptr || lds_bytes == nullptr)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "grid, block and lds_bytes must not be NULL");
  const rssm::KernelEntry* k = find_kernel(desc, 1);
  if (k == nullptr) return fail(RSSM_ERR_UNSUPPORTED, "no compiled instance");
  int g = 0;
  if (desc->max_workgroups > 0) {
    g = desc->max_workgroups;
  } else {
    st = materialize_grid(desc, k->fn, &g);
    if (st != RSSM_OK) return st;
  }
  const int lds = lds_bytes_of(k->fn);
  if (lds < 0) return fail(RSSM_ERR_HIP, "hipFuncGetAttributes failed for %s", k->name);
  *grid = g;
  *block = rssm::kBlock;
  *lds_bytes = lds;
  return RSSM_OK;
}

rssm_status rssm_materialize(const rssm_materialize_desc* desc, const rssm_materialize_tables* tables,
                             void* hip_stream) {
  g_err[0] = '\0';
  return launch(desc, tables, 1, hip_stream);
}

rssm_status rssm_materialize_checkpoints(const rssm_materialize_desc* desc, const rssm_materialize_tables* tables,
                                         int32_t num_checkpoints, void* hip_stream) {
  g_err[0] = '\0';
  if (num_checkpoints < 1 || num_checkpoints > RSSM_MAX_CHECKPOINTS)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "num_checkpoints must be in [1, %d] (got %d)", RSSM_MAX_CHECKPOINTS,
                num_checkpoints);
  return launch(desc, tables, num_checkpoints, hip_stream);
}

rssm_status rssm_gdn_commit(const rssm_gdn_commit_desc* d, const rssm_gdn_commit_tables* t, void* hip_stream) {
  g_err[0] = '\0';
  if (d == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->num_layers < 1) return fail(RSSM_ERR_INVALID_ARGUMENT, "num_layers must be >= 1 (got %d)", d->num_layers);
  if (d->slots < 1) return fail(RSSM_ERR_INVALID_ARGUMENT, "slots must be >= 1 (got %d)", d->slots);
  if (d->num_v_heads < 1 || d->num_k_heads < 1 || d->num_v_heads % d->num_k_heads != 0)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "num_k_heads (%d) must be >= 1 and divide num_v_heads (%d)",
                d->num_k_heads, d->num_v_heads);
  if (d->window < 1 || d->window > 16)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "window must be in [1, 16] (got %d)", d->window);
  if (d->batch < 0) return fail(RSSM_ERR_INVALID_ARGUMENT, "batch must be >= 0 (got %d)", d->batch);
  if (d->use_l2norm != 0 && d->use_l2norm != 1)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "use_l2norm must be 0 or 1 (got %d)", d->use_l2norm);
  if (d->null_block_id < -1)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "null_block_id must be >= -1 (got %d)", d->null_block_id);
  if (d->max_workgroups < 0)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "max_workgroups must be >= 0 (got %d)", d->max_workgroups);
  const int64_t tiles = static_cast<int64_t>(d->num_layers) * d->slots * d->num_v_heads;
  if (tiles > (int64_t(1) << 40))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "num_layers*slots*num_v_heads = %lld exceeds 2^40",
                static_cast<long long>(tiles));
  if (static_cast<int64_t>(d->batch) * d->num_layers * d->num_v_heads > (int64_t(1) << 40))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "batch*num_layers*num_v_heads exceeds 2^40");
  if (t == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "tables is NULL");
  struct P { const void* p; const char* n; int align; };
  const P ptrs[] = {{t->checkpoint_state, "checkpoint_state", 16}, {t->rawv_cache, "rawv_cache", 16},
                    {t->rawk_cache, "rawk_cache", 16}, {t->g_cache, "g_cache", 4}, {t->beta_cache, "beta_cache", 4},
                    {t->state_indices, "state_indices", 4}, {t->accept_lens, "accept_lens", 4}};
  for (const P& e : ptrs) {
    if (e.p == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "%s is NULL", e.n);
    if (!aligned(e.p, e.align)) return fail(RSSM_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", e.n, e.align);
  }
  if ((t->track_state_indices == nullptr) != (t->track_steps == nullptr))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "track_state_indices and track_steps go together (both or neither)");
  if (t->track_state_indices != nullptr && (!aligned(t->track_state_indices, 4) || !aligned(t->track_steps, 4)))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "track tables are not 4-byte aligned");
  if (d->batch == 0) return RSSM_OK;
  const void* fn = rssm::gdn_kernel_for(d->window);
  int grid = d->max_workgroups;
  if (grid == 0) {
    rssm_status st = grid_for(fn, &grid);
    if (st != RSSM_OK) return st;
  }
  rssm::GdnArgs args;
  args.state = t->checkpoint_state;
  args.rawv = t->rawv_cache;
  args.rawk = t->rawk_cache;
  args.g = t->g_cache;
  args.beta = t->beta_cache;
  args.state_indices = t->state_indices;
  args.accept_lens = t->accept_lens;
  args.track_indices = t->track_state_indices;
  args.track_steps = t->track_steps;
  args.L = d->num_layers;
  args.slots = d->slots;
  args.HV = d->num_v_heads;
  args.H = d->num_k_heads;
  args.T = d->window;
  args.B = d->batch;
  args.use_l2norm = d->use_l2norm;
  args.null_block_id = d->null_block_id;
  if (verbose())
    std::fprintf(stderr, "[rssm_gdn_commit] window<=%d grid=%d block=%d L=%d B=%d HV=%d H=%d\n",
                 d->window <= 8 ? 8 : 16, grid, rssm::kBlock, d->num_layers, d->batch, d->num_v_heads,
                 d->num_k_heads);
  void* params[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(rssm::kBlock), params, 0, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(RSSM_ERR_HIP, "launch of gdn_commit failed: %s", hipGetErrorString(e));
  return RSSM_OK;
}

rssm_status rssm_ssu_decode(const rssm_ssu_decode_desc* d, const rssm_ssu_decode_tables* t, void* hip_stream) {
  g_err[0] = '\0';
  if (d == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 0) return fail(RSSM_ERR_INVALID_ARGUMENT, "batch must be >= 0 (got %d)", d->batch);
  if (d->num_heads < 1) return fail(RSSM_ERR_INVALID_ARGUMENT, "num_heads must be >= 1 (got %d)", d->num_heads);
  if (d->heads_per_group < 1 || d->num_heads % d->heads_per_group != 0)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "heads_per_group (%d) must be >= 1 and divide num_heads (%d)",
                d->heads_per_group, d->num_heads);
  if (d->tokens < 1 || d->tokens > RSSM_SSU_MAX_TOKENS)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "tokens must be in [1, %d] (got %d)", RSSM_SSU_MAX_TOKENS, d->tokens);
  if (d->ring_buffer_len < d->tokens)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "ring_buffer_len (%d) must be >= tokens (%d)", d->ring_buffer_len,
                d->tokens);
  if (d->num_slots < 1) return fail(RSSM_ERR_INVALID_ARGUMENT, "num_slots must be >= 1 (got %d)", d->num_slots);
  if (d->dt_softplus != 0 && d->dt_softplus != 1)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "dt_softplus must be 0 or 1 (got %d)", d->dt_softplus);
  if (d->max_workgroups < 0)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "max_workgroups must be >= 0 (got %d)", d->max_workgroups);
  for (int dt : {d->state_dtype, d->input_dtype})
    if (dt < RSSM_F32 || dt > RSSM_F8E4M3) return fail(RSSM_ERR_INVALID_ARGUMENT, "unknown dtype %d", dt);
  if (d->state_dtype > RSSM_F16 || d->input_dtype > RSSM_F16)
    return fail(RSSM_ERR_UNSUPPORTED, "state and input dtypes must be f32, bf16 or f16 (got %s, %s)",
                dtype_name(d->state_dtype), dtype_name(d->input_dtype));
  if (d->dim != rssm::kSsuDim || d->dstate != rssm::kSsuDstate)
    return fail(RSSM_ERR_UNSUPPORTED, "no compiled instance for dim=%d dstate=%d (64, 128)", d->dim, d->dstate);
  const int64_t H = d->num_heads, G = H / d->heads_per_group, R = d->ring_buffer_len;
  const int64_t sb = (d->state_dtype == RSSM_F32) ? 4 : 2, ib = (d->input_dtype == RSSM_F32) ? 4 : 2;
  // 32-bit byte offsets inside one slot's x ring
  if (R * H * d->dim * ib > (int64_t(1) << 31))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "ring_buffer_len*num_heads*dim*element size exceeds 2^31 bytes");
  if (H > (int64_t(1) << 24)) return fail(RSSM_ERR_INVALID_ARGUMENT, "num_heads exceeds 2^24");
  if (static_cast<int64_t>(d->batch) * d->tokens * H * d->dim > (int64_t(1) << 46))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "batch*tokens*num_heads*dim exceeds 2^46");
  if (d->state_slot_stride < H * d->dim * d->dstate || d->x_slot_stride < R * H * d->dim ||
      d->B_slot_stride < R * G * d->dstate || d->dt_slot_stride < R * H)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "a slot stride is below the dense per-slot size");
  if ((d->state_slot_stride * sb) % 16 != 0 || (d->B_slot_stride * ib) % 16 != 0)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "state and B slot strides must be multiples of 16 bytes");
  const int64_t max_stride = std::max(std::max(d->state_slot_stride, d->x_slot_stride),
                                      std::max(d->B_slot_stride, d->dt_slot_stride));
  if (static_cast<int64_t>(d->num_slots) * max_stride > (int64_t(1) << 46))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "num_slots*slot stride exceeds 2^46 elements");
  if (t == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "tables is NULL");
  if (d->batch == 0) return RSSM_OK;   // nothing to enqueue; empty tensors may have NULL addresses
  struct P { const void* p; const char* n; int align; };
  const P ptrs[] = {{t->state, "state", 16},       {t->x_ring, "x_ring", static_cast<int>(ib)},
                    {t->B_ring, "B_ring", 16},     {t->dt_ring, "dt_ring", 4},
                    {t->A, "A", 4},                {t->x_new, "x_new", static_cast<int>(ib)},
                    {t->B_new, "B_new", 16},       {t->C_new, "C_new", 16},
                    {t->dt_new, "dt_new", 4},      {t->y, "y", 4},
                    {t->slots, "slots", 4},        {t->ring_start, "ring_start", 4},
                    {t->num_buffered, "num_buffered", 4}};
  for (const P& e : ptrs) {
    if (e.p == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "%s is NULL", e.n);
    if (!aligned(e.p, e.align)) return fail(RSSM_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", e.n, e.align);
  }
  const P opt[] = {{t->D, "D", 4}, {t->dt_bias, "dt_bias", 4}, {t->z, "z", static_cast<int>(ib)}};
  for (const P& e : opt)
    if (e.p != nullptr && !aligned(e.p, e.align))
      return fail(RSSM_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", e.n, e.align);
  const void* fn = rssm::ssu_kernel_for(d->state_dtype, d->input_dtype, d->tokens);
  if (fn == nullptr) return fail(RSSM_ERR_UNSUPPORTED, "no decode-step instance for these dtypes and tokens");
  int grid = d->max_workgroups;
  if (grid == 0) {
    // One (request, head) item per wavefront, up to 16 times the resident
    // capacity: measured on MI355X (ssu_large), a grid that streams items in
    // launch order ran 13% faster than the persistent one (0.222 against
    // 0.255 ms): the tiles in flight at any moment then lie close together.
    int resident = 0;
    rssm_status st = grid_for(fn, &resident);
    if (st != RSSM_OK) return st;
    const int64_t items = static_cast<int64_t>(d->batch) * d->num_heads;
    const int64_t want = (items + rssm::kWaves - 1) / rssm::kWaves;
    grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(want, int64_t(16) * resident)));
  }
  rssm::SsuArgs args;
  args.state = static_cast<const char*>(t->state);
  args.x_ring = static_cast<char*>(t->x_ring);
  args.B_ring = static_cast<char*>(t->B_ring);
  args.dt_ring = t->dt_ring;
  args.A = t->A;
  // absent optional vectors: the kernel reads A in their place and ignores it
  args.D = t->D != nullptr ? t->D : t->A;
  args.dt_bias = t->dt_bias != nullptr ? t->dt_bias : t->A;
  args.x_new = static_cast<const char*>(t->x_new);
  args.B_new = static_cast<const char*>(t->B_new);
  args.C_new = static_cast<const char*>(t->C_new);
  args.dt_new = t->dt_new;
  args.z = static_cast<const char*>(t->z != nullptr ? t->z : t->x_new);
  args.y = t->y;
  args.slots = t->slots;
  args.ring_start = t->ring_start;
  args.num_buffered = t->num_buffered;
  args.state_stride = d->state_slot_stride;
  args.x_stride = d->x_slot_stride;
  args.B_stride = d->B_slot_stride;
  args.dt_stride = d->dt_slot_stride;
  args.B = d->batch;
  args.H = d->num_heads;
  args.hpg = d->heads_per_group;
  args.R = d->ring_buffer_len;
  args.T = d->tokens;
  args.pad = d->pad_slot_id;
  args.num_slots = d->num_slots;
  args.dt_softplus = d->dt_softplus;
  args.has_D = t->D != nullptr;
  args.has_bias = t->dt_bias != nullptr;
  args.has_z = t->z != nullptr;
  if (verbose())
    std::fprintf(stderr, "[rssm_ssu_decode] %s/%s tokens<=%d grid=%d block=%d B=%d H=%d\n",
                 dtype_name(d->state_dtype), dtype_name(d->input_dtype), d->tokens <= 4 ? 4 : 8, grid,
                 rssm::kBlock, d->batch, d->num_heads);
  void* params[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(rssm::kBlock), params, 0, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(RSSM_ERR_HIP, "launch of ssu_decode failed: %s", hipGetErrorString(e));
  return RSSM_OK;
}

rssm_status rssm_debug_encode_rows(const rssm_materialize_desc* desc, const float* rows, const int32_t* coords,
                                   const int64_t* rand_seed, void* out_codes, float* out_scales, int32_t n,
                                   void* hip_stream) {
  g_err[0] = '\0';
  if (desc == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (desc->state_dtype < RSSM_F32 || desc->state_dtype > RSSM_F8E4M3)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "unknown state_dtype %d", desc->state_dtype);
  if (desc->philox_rounds < 0 || desc->philox_rounds > 64)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "philox_rounds must be in [0, 64]");
  if (n < 0) return fail(RSSM_ERR_INVALID_ARGUMENT, "n must be >= 0");
  const bool ob = one_byte(desc->state_dtype);
  if (!(desc->dstate == 128 || (!ob && desc->dstate == 16)))
    return fail(RSSM_ERR_UNSUPPORTED, "dstate %d not supported for %s rows", desc->dstate,
                dtype_name(desc->state_dtype));
  if (n == 0) return RSSM_OK;
  if (rows == nullptr || out_codes == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "rows/out_codes NULL");
  if (ob && out_scales == nullptr) return fail(RSSM_ERR_INVALID_ARGUMENT, "out_scales NULL for one-byte state");
  if (desc->philox_rounds > 0 && (rand_seed == nullptr || coords == nullptr))
    return fail(RSSM_ERR_INVALID_ARGUMENT, "rand_seed and coords are required when philox_rounds > 0");
  const rssm::EncodeEntry* e = find_encoder(desc);
  if (e == nullptr) return fail(RSSM_ERR_UNSUPPORTED, "no compiled encode instance");
  const int rows_per_block = rssm::kWaves * (64 / (desc->dstate / 8));
  const int grid = static_cast<int>((static_cast<int64_t>(n) + rows_per_block - 1) / rows_per_block);
  int rounds = desc->philox_rounds;
  char* codes = static_cast<char*>(out_codes);
  void* params[] = {&rows, &coords, &rand_seed, &codes, &out_scales, &n, &rounds};
  hipError_t err = hipLaunchKernel(e->fn, dim3(grid), dim3(rssm::kBlock), params, 0,
                                   static_cast<hipStream_t>(hip_stream));
  if (err != hipSuccess) return fail(RSSM_ERR_HIP, "launch of %s failed: %s", e->name, hipGetErrorString(err));
  return RSSM_OK;
}

rssm_status rssm_debug_row_scales(int32_t state_dtype, const float* rowmax, float* scale, float* inv, int32_t n,
                                  void* hip_stream) {
  g_err[0] = '\0';
  if (state_dtype != RSSM_I8 && state_dtype != RSSM_F8E4M3)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "state_dtype must be a one-byte state (I8 or F8E4M3), got %d",
                state_dtype);
  if (n < 0) return fail(RSSM_ERR_INVALID_ARGUMENT, "n must be >= 0");
  if (n == 0) return RSSM_OK;
  if (rowmax == nullptr || scale == nullptr || inv == nullptr)
    return fail(RSSM_ERR_INVALID_ARGUMENT, "rowmax, scale and inv must not be NULL");
  const void* fn = state_dtype == RSSM_I8 ? reinterpret_cast<const void*>(&rssm::row_scales_kernel<127>)
                                          : reinterpret_cast<const void*>(&rssm::row_scales_kernel<448>);
  const int grid = static_cast<int>((static_cast<int64_t>(n) + rssm::kBlock - 1) / rssm::kBlock);
  void* params[] = {&rowmax, &scale, &inv, &n};
  hipError_t err = hipLaunchKernel(fn, dim3(grid), dim3(rssm::kBlock), params, 0,
                                   static_cast<hipStream_t>(hip_stream));
  if (err != hipSuccess) return fail(RSSM_ERR_HIP, "launch of row_scales_kernel failed: %s", hipGetErrorString(err));
  return RSSM_OK;
}

}  // extern "C"
