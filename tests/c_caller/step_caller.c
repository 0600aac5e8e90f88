/*
 * step_caller.c -- drives the decode step (rssm_ssu_decode) and the
 * gated-delta-rule commit (rssm_gdn_commit) of librssm_materialize from plain
 * C, through their headers and the HIP runtime alone (no Python, no torch).
 * Test infrastructure: it computes nothing of the method itself.
 *
 * Usage: step_caller ssu|gdn DIR
 *
 * DIR/desc.txt holds "name value" lines, one per field of the call's
 * descriptor (rssm_ssu_decode_desc or rssm_gdn_commit_desc, integers).
 * DIR/<field>.bin holds the raw little-endian bytes of each device tensor of
 * the call's tables, named as the fields of rssm_ssu_decode_tables or
 * rssm_gdn_commit_tables; an optional tensor whose file is absent is passed as
 * NULL.  The program checks every size and the device-metadata contract on
 * the host before any HIP call, uploads each tensor to an allocation of its
 * own, makes the call on a stream it creates, waits for it, checks that the
 * tensors the call only reads came back unchanged, and writes <field>.out
 * for each tensor the call writes (ssu: x_ring B_ring dt_ring y; gdn:
 * checkpoint_state).
 *
 * Exit status: 0 done; 1 usage, file or host-check error; 2 a library status
 * other than RSSM_OK; 3 a HIP runtime error; 4 the call changed a tensor it
 * only reads.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rssm_gdn_commit.h"
#include "rssm_materialize.h"
#include "rssm_ssu_decode.h"

static const char *g_dir;

static void die(int code, const char *what, const char *detail) {
  fprintf(stderr, "step_caller: %s%s%s\n", what, detail ? ": " : "", detail ? detail : "");
  exit(code);
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) die(3, #call, hipGetErrorString(e_));        \
  } while (0)

typedef struct {
  const char *name;
  int required, written;
  size_t want;  /* bytes the call's shapes give this tensor */
  void *host, *dev;
  size_t bytes;
} tensor;

static void path_of(char *out, size_t n, const char *name, const char *ext) {
  int w = snprintf(out, n, "%s/%s.%s", g_dir, name, ext);
  if (w < 0 || (size_t)w >= n) die(1, "path too long for", name);
}

/* Read DIR/<name>.bin into host memory; an absent optional file leaves the
 * tensor empty (passed as NULL). */
static void load(tensor *t) {
  char path[4096];
  path_of(path, sizeof path, t->name, "bin");
  FILE *f = fopen(path, "rb");
  if (!f) {
    if (t->required) die(1, "cannot open", path);
    return;
  }
  if (fseek(f, 0, SEEK_END) != 0) die(1, "cannot seek", path);
  long sz = ftell(f);
  if (sz < 0 || fseek(f, 0, SEEK_SET) != 0) die(1, "cannot size", path);
  t->bytes = (size_t)sz;
  t->host = malloc(t->bytes ? t->bytes : 1);
  if (!t->host) die(1, "out of host memory for", path);
  if (t->bytes && fread(t->host, 1, t->bytes, f) != t->bytes) die(1, "short read", path);
  fclose(f);
  if (t->bytes != t->want) {
    fprintf(stderr, "step_caller: %s has %zu bytes, the shapes give %zu\n", t->name, t->bytes, t->want);
    exit(1);
  }
}

static void upload(tensor *t) {
  if (!t->host) return;
  HIP_OK(hipMalloc(&t->dev, t->bytes ? t->bytes : 16));
  if (t->bytes) HIP_OK(hipMemcpy(t->dev, t->host, t->bytes, hipMemcpyHostToDevice));
}

static void finish(tensor *t) {
  if (!t->host) return;
  void *h = malloc(t->bytes ? t->bytes : 1);
  if (!h) die(1, "out of host memory", NULL);
  if (t->bytes) HIP_OK(hipMemcpy(h, t->dev, t->bytes, hipMemcpyDeviceToHost));
  if (t->written) {
    char path[4096];
    path_of(path, sizeof path, t->name, "out");
    FILE *f = fopen(path, "wb");
    if (!f) die(1, "cannot create", path);
    if (t->bytes && fwrite(h, 1, t->bytes, f) != t->bytes) die(1, "short write", path);
    if (fclose(f) != 0) die(1, "cannot close", path);
  } else if (t->bytes && memcmp(h, t->host, t->bytes) != 0) {
    die(4, "the call changed a tensor it only reads", t->name);
  }
  free(h);
  HIP_OK(hipFree(t->dev));
  free(t->host);
}

/* desc.txt: "name value" lines; every name asked for must be present. */
typedef struct {
  char name[64];
  long long value;
} field;
static field g_fields[64];
static int g_nfields;

static void read_desc(void) {
  char path[4096];
  path_of(path, sizeof path, "desc", "txt");
  FILE *f = fopen(path, "r");
  if (!f) die(1, "cannot open", path);
  while (g_nfields < 64 && fscanf(f, "%63s %lld", g_fields[g_nfields].name, &g_fields[g_nfields].value) == 2)
    ++g_nfields;
  fclose(f);
}

static long long get(const char *name) {
  for (int i = 0; i < g_nfields; ++i)
    if (strcmp(g_fields[i].name, name) == 0) return g_fields[i].value;
  die(1, "desc.txt lacks", name);
  return 0;
}

static int32_t get32(const char *name) {
  long long v = get(name);
  if (v < INT32_MIN || v > INT32_MAX) die(1, "desc value out of int32 range", name);
  return (int32_t)v;
}

static size_t elem(int32_t dtype) {
  switch (dtype) {
    case RSSM_F32: return 4;
    case RSSM_BF16: case RSSM_F16: return 2;
    default: die(1, "unsupported dtype in desc.txt", NULL);
  }
  return 0;
}

static size_t positive(long long v, const char *what) {
  if (v < 1) die(1, "desc value must be positive", what);
  return (size_t)v;
}

static void call_status(rssm_status st, const char *what) {
  if (st != RSSM_OK) die(2, what, rssm_last_error());
}

static int run_ssu(void) {
  rssm_ssu_decode_desc d;
  memset(&d, 0, sizeof d);
  d.batch = get32("batch");
  d.num_heads = get32("num_heads");
  d.heads_per_group = get32("heads_per_group");
  d.dim = get32("dim");
  d.dstate = get32("dstate");
  d.ring_buffer_len = get32("ring_buffer_len");
  d.tokens = get32("tokens");
  d.num_slots = get32("num_slots");
  d.pad_slot_id = get32("pad_slot_id");
  d.state_dtype = get32("state_dtype");
  d.input_dtype = get32("input_dtype");
  d.dt_softplus = get32("dt_softplus");
  d.max_workgroups = get32("max_workgroups");
  d.state_slot_stride = get("state_slot_stride");
  d.x_slot_stride = get("x_slot_stride");
  d.B_slot_stride = get("B_slot_stride");
  d.dt_slot_stride = get("dt_slot_stride");

  const size_t B = positive(d.batch, "batch"), H = positive(d.num_heads, "num_heads");
  const size_t hpg = positive(d.heads_per_group, "heads_per_group");
  if (H % hpg) die(1, "heads_per_group must divide num_heads", NULL);
  const size_t G = H / hpg, dim = positive(d.dim, "dim"), ds = positive(d.dstate, "dstate");
  const size_t T = positive(d.tokens, "tokens"), S = positive(d.num_slots, "num_slots");
  const size_t R = positive(d.ring_buffer_len, "ring_buffer_len");
  const size_t sb = elem(d.state_dtype), ib = elem(d.input_dtype);
  if (d.state_slot_stride < (long long)(H * dim * ds) || d.x_slot_stride < (long long)(R * H * dim) ||
      d.B_slot_stride < (long long)(R * G * ds) || d.dt_slot_stride < (long long)(R * H))
    die(1, "a slot stride is below the dense slot size", NULL);

  enum { STATE, XR, BR, DTR, A, D, BIAS, XN, BN, CN, DTN, Z, Y, SLOTS, RS, NB, NT };
  tensor t[NT] = {
      {"state", 1, 0, S * (size_t)d.state_slot_stride * sb, 0, 0, 0},
      {"x_ring", 1, 1, S * (size_t)d.x_slot_stride * ib, 0, 0, 0},
      {"B_ring", 1, 1, S * (size_t)d.B_slot_stride * ib, 0, 0, 0},
      {"dt_ring", 1, 1, S * (size_t)d.dt_slot_stride * 4, 0, 0, 0},
      {"A", 1, 0, H * 4, 0, 0, 0},
      {"D", 0, 0, H * 4, 0, 0, 0},
      {"dt_bias", 0, 0, H * 4, 0, 0, 0},
      {"x_new", 1, 0, B * T * H * dim * ib, 0, 0, 0},
      {"B_new", 1, 0, B * T * G * ds * ib, 0, 0, 0},
      {"C_new", 1, 0, B * T * G * ds * ib, 0, 0, 0},
      {"dt_new", 1, 0, B * T * H * 4, 0, 0, 0},
      {"z", 0, 0, B * T * H * dim * ib, 0, 0, 0},
      {"y", 1, 1, B * T * H * dim * 4, 0, 0, 0},
      {"slots", 1, 0, B * 4, 0, 0, 0},
      {"ring_start", 1, 0, B * 4, 0, 0, 0},
      {"num_buffered", 1, 0, B * 4, 0, 0, 0},
  };
  for (int i = 0; i < NT; ++i) load(&t[i]);

  /* the device-metadata contract, checked here because the library does not */
  const int32_t *sl = (const int32_t *)t[SLOTS].host, *rs = (const int32_t *)t[RS].host;
  const int32_t *nb = (const int32_t *)t[NB].host;
  const long long cap = R < RSSM_SSU_MAX_REPLAY ? (long long)R : RSSM_SSU_MAX_REPLAY;
  for (size_t b = 0; b < B; ++b) {
    if (sl[b] == d.pad_slot_id) continue;
    if (sl[b] < 0 || (size_t)sl[b] >= S) die(1, "a live slot lies outside the pool", NULL);
    for (size_t c = 0; c < b; ++c)
      if (sl[c] == sl[b]) die(1, "two live requests share a slot", NULL);
    if (rs[b] < 0 || (size_t)rs[b] >= R) die(1, "ring_start outside [0, R)", NULL);
    if (nb[b] < 0 || nb[b] + (long long)T > cap) die(1, "num_buffered outside the contract", NULL);
  }

  for (int i = 0; i < NT; ++i) upload(&t[i]);
  rssm_ssu_decode_tables tab;
  memset(&tab, 0, sizeof tab);
  tab.state = t[STATE].dev;
  tab.x_ring = t[XR].dev;
  tab.B_ring = t[BR].dev;
  tab.dt_ring = (float *)t[DTR].dev;
  tab.A = (const float *)t[A].dev;
  tab.D = (const float *)t[D].dev;
  tab.dt_bias = (const float *)t[BIAS].dev;
  tab.x_new = t[XN].dev;
  tab.B_new = t[BN].dev;
  tab.C_new = t[CN].dev;
  tab.dt_new = (const float *)t[DTN].dev;
  tab.z = t[Z].dev;
  tab.y = (float *)t[Y].dev;
  tab.slots = (const int32_t *)t[SLOTS].dev;
  tab.ring_start = (const int32_t *)t[RS].dev;
  tab.num_buffered = (const int32_t *)t[NB].dev;

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  call_status(rssm_ssu_decode(&d, &tab, (void *)stream), "rssm_ssu_decode");
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipStreamDestroy(stream));
  printf("ssu ok\n");
  for (int i = 0; i < NT; ++i) finish(&t[i]);
  return 0;
}

static int run_gdn(void) {
  rssm_gdn_commit_desc d;
  memset(&d, 0, sizeof d);
  d.num_layers = get32("num_layers");
  d.slots = get32("slots");
  d.num_v_heads = get32("num_v_heads");
  d.num_k_heads = get32("num_k_heads");
  d.window = get32("window");
  d.batch = get32("batch");
  d.use_l2norm = get32("use_l2norm");
  d.null_block_id = get32("null_block_id");
  d.max_workgroups = get32("max_workgroups");

  const size_t L = positive(d.num_layers, "num_layers"), S = positive(d.slots, "slots");
  const size_t HV = positive(d.num_v_heads, "num_v_heads"), H = positive(d.num_k_heads, "num_k_heads");
  const size_t T = positive(d.window, "window"), B = positive(d.batch, "batch");
  if (HV % H) die(1, "num_k_heads must divide num_v_heads", NULL);

  enum { ST, V, K, GC, BETA, IDX, ACC, TIDX, TSTEP, NT };
  tensor t[NT] = {
      {"checkpoint_state", 1, 1, L * S * HV * 128 * 128 * 4, 0, 0, 0},
      {"rawv_cache", 1, 0, L * S * HV * T * 128 * 2, 0, 0, 0},
      {"rawk_cache", 1, 0, L * S * H * T * 128 * 2, 0, 0, 0},
      {"g_cache", 1, 0, L * S * HV * T * 4, 0, 0, 0},
      {"beta_cache", 1, 0, L * S * HV * T * 4, 0, 0, 0},
      {"state_indices", 1, 0, B * 4, 0, 0, 0},
      {"accept_lens", 1, 0, B * 4, 0, 0, 0},
      {"track_state_indices", 0, 0, B * 4, 0, 0, 0},
      {"track_steps", 0, 0, B * 4, 0, 0, 0},
  };
  for (int i = 0; i < NT; ++i) load(&t[i]);
  if (!t[TIDX].host != !t[TSTEP].host) die(1, "track_state_indices and track_steps come together", NULL);

  /* the device-metadata contract, checked here because the library does not */
  const int32_t *idx = (const int32_t *)t[IDX].host, *acc = (const int32_t *)t[ACC].host;
  const int32_t *tidx = (const int32_t *)t[TIDX].host;
  for (size_t b = 0; b < B; ++b) {
    if (acc[b] < 0 || (size_t)acc[b] > T) die(1, "accept_lens outside [0, T]", NULL);
    const int live = idx[b] > d.null_block_id;
    if (live && (size_t)idx[b] >= S) die(1, "a live slot lies outside the pool", NULL);
    if (tidx && tidx[b] > d.null_block_id && (size_t)tidx[b] >= S) die(1, "a track slot lies outside the pool", NULL);
    for (size_t c = 0; c < b; ++c) {
      if (live && idx[c] == idx[b]) die(1, "two live requests share a slot", NULL);
      if (tidx && tidx[b] > d.null_block_id && tidx[c] == tidx[b]) die(1, "two track slots coincide", NULL);
    }
    if (tidx && tidx[b] > d.null_block_id)
      for (size_t c = 0; c < B; ++c)
        if (idx[c] > d.null_block_id && idx[c] == tidx[b]) die(1, "a track slot is a live state slot", NULL);
  }

  for (int i = 0; i < NT; ++i) upload(&t[i]);
  rssm_gdn_commit_tables tab;
  memset(&tab, 0, sizeof tab);
  tab.checkpoint_state = (float *)t[ST].dev;
  tab.rawv_cache = (const uint16_t *)t[V].dev;
  tab.rawk_cache = (const uint16_t *)t[K].dev;
  tab.g_cache = (const float *)t[GC].dev;
  tab.beta_cache = (const float *)t[BETA].dev;
  tab.state_indices = (const int32_t *)t[IDX].dev;
  tab.accept_lens = (const int32_t *)t[ACC].dev;
  tab.track_state_indices = (const int32_t *)t[TIDX].dev;
  tab.track_steps = (const int32_t *)t[TSTEP].dev;

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  call_status(rssm_gdn_commit(&d, &tab, (void *)stream), "rssm_gdn_commit");
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipStreamDestroy(stream));
  printf("gdn ok\n");
  for (int i = 0; i < NT; ++i) finish(&t[i]);
  return 0;
}

int main(int argc, char **argv) {
  if (argc != 3) die(1, "usage", "step_caller ssu|gdn DIR");
  g_dir = argv[2];
  read_desc();
  if (strcmp(argv[1], "ssu") == 0) return run_ssu();
  if (strcmp(argv[1], "gdn") == 0) return run_gdn();
  die(1, "unknown call", argv[1]);
  return 1;
}
