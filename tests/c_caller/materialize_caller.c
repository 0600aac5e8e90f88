/*
 * materialize_caller.c -- drives librssm_materialize from plain C through
 * rssm_materialize.h and the HIP runtime alone (no Python, no torch), so that
 * a test can show the boundary stands on its own.  Test infrastructure: it
 * computes nothing of the method itself.
 *
 * Usage: materialize_caller DIR [EMPTY_CALLS]
 *
 * DIR/problem.txt holds whitespace-separated integers:
 *   num_layers batch num_heads heads_per_group dim dstate max_window
 *   ring_buffer_len pad_slot_id philox_rounds state_dtype input_dtype
 *   max_workgroups has_scale has_seed num_checkpoints
 * followed, for each layer, by its slot strides in elements:
 *   state scale x B dt
 * DIR also holds one raw little-endian blob per buffer (the layouts of
 * rssm_materialize.h):
 *   state_<l>.bin x_<l>.bin B_<l>.bin dt_<l>.bin A_<l>.bin [scale_<l>.bin]
 *   src.bin dst.bin ([L][B] int32)  ring_start.bin prefix.bin active.bin
 *   ([B] int32)  [seed.bin (one int64)]
 * num_checkpoints 0 makes one rssm_materialize call; C >= 1 makes one
 * rssm_materialize_checkpoints call with C tables: dst.bin then holds
 * [C][L][B] and prefix.bin [C][B] int32.
 *
 * The program reads every blob, checks on the host (before any HIP call) that
 * every slot the call will touch lies inside its pool, uploads each blob to a
 * device allocation of its own, builds the pointer and stride tables, prints
 * the launch the library would make, checks that an invalid descriptor is
 * refused with a message, makes the call on a stream it creates, waits for it, checks that the rings, A and the metadata came back
 * unchanged, and writes state_<l>.out (and scale_<l>.out) with the pools as
 * the call left them.
 *
 * With EMPTY_CALLS > 0 it then also times that many back-to-back calls whose
 * active list is empty (every entry -1) on the same stream, after as many
 * untimed ones, with HIP events, and prints "empty_call_us <mean>": the cost
 * of a call with nothing to do, host side included, with no Python involved.
 *
 * Exit status: 0 done; 1 usage, file or host-check error; 2 a library status
 * other than the one expected; 3 a HIP runtime error; 4 the call changed a
 * buffer it only reads.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rssm_materialize.h"

#define MAX_LAYERS 1024

static const char *g_dir;

static void die(int code, const char *what, const char *detail) {
  fprintf(stderr, "materialize_caller: %s%s%s\n", what, detail ? ": " : "", detail ? detail : "");
  exit(code);
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) die(3, #call, hipGetErrorString(e_));        \
  } while (0)

typedef struct {
  void *host;
  void *dev;
  size_t bytes;
} blob;

static void path_of(char *out, size_t n, const char *name, int layer, const char *ext) {
  int w = layer >= 0 ? snprintf(out, n, "%s/%s_%d.%s", g_dir, name, layer, ext)
                     : snprintf(out, n, "%s/%s.%s", g_dir, name, ext);
  if (w < 0 || (size_t)w >= n) die(1, "path too long for", name);
}

static void *device_copy(const void *host, size_t bytes) {
  void *dev = NULL;
  HIP_OK(hipMalloc(&dev, bytes ? bytes : 16));
  if (bytes) HIP_OK(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice));
  return dev;
}

/* Read DIR/name[_layer].bin into host memory.  Returns 0 (and an empty
 * blob) when the file is absent and not required. */
static int load(const char *name, int layer, int required, blob *b) {
  char path[4096];
  path_of(path, sizeof path, name, layer, "bin");
  memset(b, 0, sizeof *b);
  FILE *f = fopen(path, "rb");
  if (!f) {
    if (required) die(1, "cannot open", path);
    return 0;
  }
  if (fseek(f, 0, SEEK_END) != 0) die(1, "cannot seek", path);
  long sz = ftell(f);
  if (sz < 0 || fseek(f, 0, SEEK_SET) != 0) die(1, "cannot size", path);
  b->bytes = (size_t)sz;
  b->host = malloc(b->bytes ? b->bytes : 1);
  if (!b->host) die(1, "out of host memory for", path);
  if (b->bytes && fread(b->host, 1, b->bytes, f) != b->bytes) die(1, "short read", path);
  fclose(f);
  return 1;
}

static void upload(blob *b) {
  if (b->host) b->dev = device_copy(b->host, b->bytes);
}

static void save(const char *name, int layer, const blob *b) {
  char path[4096];
  path_of(path, sizeof path, name, layer, "out");
  void *h = malloc(b->bytes ? b->bytes : 1);
  if (!h) die(1, "out of host memory for", path);
  if (b->bytes) HIP_OK(hipMemcpy(h, b->dev, b->bytes, hipMemcpyDeviceToHost));
  FILE *f = fopen(path, "wb");
  if (!f) die(1, "cannot create", path);
  if (b->bytes && fwrite(h, 1, b->bytes, f) != b->bytes) die(1, "short write", path);
  if (fclose(f) != 0) die(1, "cannot close", path);
  free(h);
}

/* 1 when the device copy still holds the bytes that were uploaded. */
static int unchanged(const blob *b) {
  if (!b->bytes) return 1;
  void *h = malloc(b->bytes);
  if (!h) die(1, "out of host memory", NULL);
  HIP_OK(hipMemcpy(h, b->dev, b->bytes, hipMemcpyDeviceToHost));
  int same = memcmp(h, b->host, b->bytes) == 0;
  free(h);
  return same;
}

static void release(blob *b) {
  if (b->dev) HIP_OK(hipFree(b->dev));
  free(b->host);
  memset(b, 0, sizeof *b);
}

static size_t elem_bytes(int32_t dtype) {
  switch (dtype) {
    case RSSM_F32: return 4;
    case RSSM_BF16: case RSSM_F16: return 2;
    case RSSM_I8: case RSSM_F8E4M3: return 1;
    default: die(1, "unknown dtype in problem.txt", NULL);
  }
  return 0;
}

/* Slots a pool of `bytes` holds at `stride` elements of `eb` bytes, or -1
 * when the blob is not a whole number of slots. */
static int64_t pool_slots(const blob *b, int64_t stride, size_t eb) {
  if (stride <= 0) return -1;
  size_t slot = (size_t)stride * eb;
  return b->bytes % slot ? -1 : (int64_t)(b->bytes / slot);
}

int main(int argc, char **argv) {
  if (argc != 2 && argc != 3) die(1, "usage", "materialize_caller DIR [EMPTY_CALLS]");
  const long empty_calls = argc == 3 ? strtol(argv[2], NULL, 10) : 0;
  if (empty_calls < 0 || empty_calls > 1000000) die(1, "EMPTY_CALLS out of range", argv[2]);
  g_dir = argv[1];

  char path[4096];
  path_of(path, sizeof path, "problem", -1, "txt");
  FILE *pf = fopen(path, "r");
  if (!pf) die(1, "cannot open", path);
  rssm_materialize_desc desc;
  memset(&desc, 0, sizeof desc);
  int has_scale = 0, has_seed = 0, ncp = 0;
  desc.a_dtype = RSSM_F32;
  if (fscanf(pf, "%d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d", &desc.num_layers, &desc.batch,
             &desc.num_heads, &desc.heads_per_group, &desc.dim, &desc.dstate, &desc.max_window,
             &desc.ring_buffer_len, &desc.pad_slot_id, &desc.philox_rounds, &desc.state_dtype,
             &desc.input_dtype, &desc.max_workgroups, &has_scale, &has_seed, &ncp) != 16)
    die(1, "malformed header in", path);
  if (ncp < 0 || ncp > RSSM_MAX_CHECKPOINTS) die(1, "num_checkpoints out of range in", path);
  const int C = ncp > 0 ? ncp : 1;  /* destination and prefix tables */
  const int L = desc.num_layers, B = desc.batch;
  if (L < 1 || L > MAX_LAYERS || B < 1 || desc.num_heads < 1 || desc.heads_per_group < 1 ||
      desc.num_heads % desc.heads_per_group)
    die(1, "problem sizes out of range in", path);
  static long long strides[5][MAX_LAYERS]; /* state scale x B dt */
  for (int l = 0; l < L; ++l)
    for (int k = 0; k < 5; ++k)
      if (fscanf(pf, "%lld", &strides[k][l]) != 1) die(1, "missing strides in", path);
  fclose(pf);

  static blob state[MAX_LAYERS], scale[MAX_LAYERS], x[MAX_LAYERS], Bm[MAX_LAYERS], dt[MAX_LAYERS],
      A[MAX_LAYERS];
  blob src, dst, ring_start, prefix, active, seed;
  for (int l = 0; l < L; ++l) {
    load("state", l, 1, &state[l]);
    load("x", l, 1, &x[l]);
    load("B", l, 1, &Bm[l]);
    load("dt", l, 1, &dt[l]);
    load("A", l, 1, &A[l]);
    if (has_scale) load("scale", l, 1, &scale[l]);
  }
  load("src", -1, 1, &src);
  load("dst", -1, 1, &dst);
  load("ring_start", -1, 1, &ring_start);
  load("prefix", -1, 1, &prefix);
  load("active", -1, 1, &active);
  if (has_seed) load("seed", -1, 1, &seed); else memset(&seed, 0, sizeof seed);
  const size_t LB = (size_t)L * B * sizeof(int32_t), B4 = (size_t)B * sizeof(int32_t);
  if (src.bytes != LB || dst.bytes != C * LB || ring_start.bytes != B4 || prefix.bytes != C * B4 ||
      active.bytes != B4 || (has_seed && seed.bytes != sizeof(int64_t)))
    die(1, "a metadata blob has the wrong size", NULL);

  /* Host checks of the device-metadata contract for the requests the call
   * will visit: the library leaves it unchecked, and a slot outside its pool
   * would be an access outside an allocation. */
  const size_t sb = elem_bytes(desc.state_dtype), ib = elem_bytes(desc.input_dtype);
  const int32_t *srcs = (const int32_t *)src.host, *dsts = (const int32_t *)dst.host;
  const int32_t *act = (const int32_t *)active.host, *pre = (const int32_t *)prefix.host;
  const int32_t *rs = (const int32_t *)ring_start.host;
  for (int i = 0; i < B && act[i] >= 0 && act[i] < B; ++i) {
    const int b = act[i];
    if (rs[b] < 0 || rs[b] >= desc.ring_buffer_len) die(1, "ring start outside the contract", NULL);
    for (int c = 0; c < C; ++c)
      if (pre[(size_t)c * B + b] < 0 || pre[(size_t)c * B + b] > desc.max_window)
        die(1, "prefix length outside the contract", NULL);
    for (int l = 0; l < L; ++l) {
      const int32_t s = srcs[(size_t)l * B + b];
      if (s == desc.pad_slot_id) continue;
      const int64_t ns = pool_slots(&state[l], strides[0][l], sb);
      const int64_t nr = pool_slots(&x[l], strides[2][l], ib);
      if (ns < 0 || nr < 0 || pool_slots(&Bm[l], strides[3][l], ib) != nr ||
          pool_slots(&dt[l], strides[4][l], 4) != nr ||
          (has_scale && pool_slots(&scale[l], strides[1][l], 4) != ns))
        die(1, "a pool is not a whole number of slots", NULL);
      if (A[l].bytes != (size_t)desc.num_heads * 4) die(1, "A has the wrong size", NULL);
      int live = 0;
      for (int c = 0; c < C; ++c) {
        const int32_t d = dsts[((size_t)c * L + l) * B + b];
        if (d == desc.pad_slot_id) continue;
        if (d < 0 || d >= ns) die(1, "a slot lies outside its pool", NULL);
        live = 1;
      }
      if (live && (s < 0 || s >= ns || s >= nr)) die(1, "a slot lies outside its pool", NULL);
    }
  }

  for (int l = 0; l < L; ++l) {
    upload(&state[l]); upload(&x[l]); upload(&Bm[l]); upload(&dt[l]); upload(&A[l]);
    upload(&scale[l]);
  }
  upload(&src); upload(&dst); upload(&ring_start); upload(&prefix); upload(&active);
  upload(&seed);

  /* Pointer and stride tables: device addresses as int64, one entry per layer. */
  static int64_t hp[6][MAX_LAYERS], hs[5][MAX_LAYERS];
  for (int l = 0; l < L; ++l) {
    hp[0][l] = (int64_t)(uintptr_t)state[l].dev;
    hp[1][l] = (int64_t)(uintptr_t)x[l].dev;
    hp[2][l] = (int64_t)(uintptr_t)Bm[l].dev;
    hp[3][l] = (int64_t)(uintptr_t)dt[l].dev;
    hp[4][l] = (int64_t)(uintptr_t)A[l].dev;
    hp[5][l] = (int64_t)(uintptr_t)scale[l].dev;
    for (int k = 0; k < 5; ++k) hs[k][l] = strides[k][l];
  }
  const size_t LT = (size_t)L * sizeof(int64_t);
  void *d_state_ptrs = device_copy(hp[0], LT), *d_x_ptrs = device_copy(hp[1], LT);
  void *d_B_ptrs = device_copy(hp[2], LT), *d_dt_ptrs = device_copy(hp[3], LT);
  void *d_A_ptrs = device_copy(hp[4], LT), *d_scale_ptrs = device_copy(hp[5], LT);
  void *d_state_str = device_copy(hs[0], LT), *d_scale_str = device_copy(hs[1], LT);
  void *d_x_str = device_copy(hs[2], LT), *d_B_str = device_copy(hs[3], LT);
  void *d_dt_str = device_copy(hs[4], LT);

  rssm_materialize_tables tab;
  memset(&tab, 0, sizeof tab);
  tab.state_ptrs = (const int64_t *)d_state_ptrs;
  tab.state_slot_strides = (const int64_t *)d_state_str;
  tab.x_ptrs = (const int64_t *)d_x_ptrs;
  tab.x_slot_strides = (const int64_t *)d_x_str;
  tab.B_ptrs = (const int64_t *)d_B_ptrs;
  tab.B_slot_strides = (const int64_t *)d_B_str;
  tab.dt_ptrs = (const int64_t *)d_dt_ptrs;
  tab.dt_slot_strides = (const int64_t *)d_dt_str;
  tab.A_ptrs = (const int64_t *)d_A_ptrs;
  tab.scale_ptrs = has_scale ? (const int64_t *)d_scale_ptrs : NULL;
  tab.scale_slot_strides = has_scale ? (const int64_t *)d_scale_str : NULL;
  tab.src_slots = (const int32_t *)src.dev;
  tab.dst_slots = (const int32_t *)dst.dev;
  tab.ring_start = (const int32_t *)ring_start.dev;
  tab.replay_prefix_len = (const int32_t *)prefix.dev;
  tab.active_request_indices = (const int32_t *)active.dev;
  tab.rand_seed = has_seed ? (const int64_t *)seed.dev : NULL;

  int32_t grid = 0, block = 0, lds = 0;
  rssm_status st = rssm_materialize_launch_config(&desc, &grid, &block, &lds);
  if (st != RSSM_OK) die(2, "rssm_materialize_launch_config", rssm_last_error());
  printf("launch grid=%d block=%d lds_bytes=%d\n", grid, block, lds);

  /* A descriptor with no layers is refused before any HIP call. */
  rssm_materialize_desc bad = desc;
  bad.num_layers = 0;
  st = rssm_materialize(&bad, &tab, NULL);
  if (st != RSSM_ERR_INVALID_ARGUMENT || rssm_last_error()[0] == '\0')
    die(2, "an empty descriptor was not refused with a message", NULL);
  printf("refused: %s\n", rssm_last_error());

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  st = ncp > 0 ? rssm_materialize_checkpoints(&desc, &tab, ncp, (void *)stream)
              : rssm_materialize(&desc, &tab, (void *)stream);
  if (st != RSSM_OK) die(2, ncp > 0 ? "rssm_materialize_checkpoints" : "rssm_materialize", rssm_last_error());
  HIP_OK(hipStreamSynchronize(stream));
  printf("materialize ok\n");

  if (empty_calls > 0) {
    /* the same call with nothing to do: every active entry -1 */
    int32_t *none = (int32_t *)malloc(B4);
    if (!none) die(1, "out of host memory", NULL);
    for (int b = 0; b < B; ++b) none[b] = -1;
    void *d_none = device_copy(none, B4);
    rssm_materialize_tables idle = tab;
    idle.active_request_indices = (const int32_t *)d_none;
    hipEvent_t e0, e1;
    HIP_OK(hipEventCreate(&e0));
    HIP_OK(hipEventCreate(&e1));
    for (long i = 0; i < empty_calls; ++i)
      if (rssm_materialize(&desc, &idle, (void *)stream) != RSSM_OK) die(2, "rssm_materialize", rssm_last_error());
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipEventRecord(e0, stream));
    for (long i = 0; i < empty_calls; ++i)
      if (rssm_materialize(&desc, &idle, (void *)stream) != RSSM_OK) die(2, "rssm_materialize", rssm_last_error());
    HIP_OK(hipEventRecord(e1, stream));
    HIP_OK(hipEventSynchronize(e1));
    float ms = 0.0f;
    HIP_OK(hipEventElapsedTime(&ms, e0, e1));
    printf("empty_call_us %.3f\n", 1000.0 * ms / (double)empty_calls);
    HIP_OK(hipEventDestroy(e0));
    HIP_OK(hipEventDestroy(e1));
    HIP_OK(hipFree(d_none));
    free(none);
  }
  HIP_OK(hipStreamDestroy(stream));

  for (int l = 0; l < L; ++l)
    if (!unchanged(&x[l]) || !unchanged(&Bm[l]) || !unchanged(&dt[l]) || !unchanged(&A[l]))
      die(4, "the call changed a ring or A", NULL);
  if (!unchanged(&src) || !unchanged(&dst) || !unchanged(&ring_start) || !unchanged(&prefix) ||
      !unchanged(&active) || !unchanged(&seed))
    die(4, "the call changed its metadata", NULL);
  for (int l = 0; l < L; ++l) {
    save("state", l, &state[l]);
    if (has_scale) save("scale", l, &scale[l]);
  }

  for (int l = 0; l < L; ++l) {
    release(&state[l]); release(&x[l]); release(&Bm[l]); release(&dt[l]); release(&A[l]);
    release(&scale[l]);
  }
  release(&src); release(&dst); release(&ring_start); release(&prefix); release(&active);
  release(&seed);
  void *tables[] = {d_state_ptrs, d_x_ptrs, d_B_ptrs, d_dt_ptrs, d_A_ptrs, d_scale_ptrs,
                    d_state_str, d_scale_str, d_x_str, d_B_str, d_dt_str};
  for (size_t i = 0; i < sizeof tables / sizeof tables[0]; ++i) HIP_OK(hipFree(tables[i]));
  printf("done\n");
  return 0;
}
