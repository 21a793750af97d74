/* One DSpark step through the C ABI of libdspark, from plain C (C99): no
 * Python, no torch.  Reads a step's inputs from a binary file, allocates its
 * own device buffers, runs dspark_draft_block, dspark_schedule and
 * dspark_verify on the default stream, gathers the verify rows on the host
 * (the stand-in for the target model's forward over the scheduled rows) and
 * writes the outputs to a second file.  tests/test_gpu_c_abi.py runs it and
 * compares its outputs with the Python binding's on the same inputs.
 *
 *   abi_step IN OUT
 *
 * IN (little-endian): int32 R, gamma, V, rank; int64 K; then
 *   float U[R][gamma][V], float target[R][gamma+1][V],
 *   uint16 W1[V][rank], uint16 W2[V][rank] (bf16 bit patterns),
 *   int32 anchor[R], float temp[R], float u_draft[R][gamma],
 *   float u_accept[R][gamma], float u_final[R], float c[R][gamma].
 * OUT: int32 y[R][gamma], float q_tok[R][gamma], float q_stats[R][gamma][2],
 *   int32 l[R], int32 row_offsets[R+1], int32 n_accept[R], int32 out_tok[R],
 *   float p_tok[R][gamma].
 * Exit status 0 on success; on any failure a message on stderr and 1. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dspark.h"

static void die(const char* what, const char* detail) {
  fprintf(stderr, "abi_step: %s: %s\n", what, detail);
  exit(1);
}

static void hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) die(what, hipGetErrorString(e));
}

static void ds_ok(int st, const char* what) {
  if (st != DSPARK_OK) die(what, dspark_status_string(st));
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  hip_ok(hipMalloc(&p, bytes ? bytes : 1), "hipMalloc");
  return p;
}

/* a device copy of n bytes read from f */
static void* dev_read(FILE* f, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (!h) die("malloc", "out of memory");
  if (bytes && fread(h, 1, bytes, f) != bytes) die("read", "input file too short");
  void* d = dev_alloc(bytes);
  hip_ok(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy H2D");
  free(h);
  return d;
}

static void host_write(FILE* f, const void* d, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (!h) die("malloc", "out of memory");
  hip_ok(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost), "hipMemcpy D2H");
  if (bytes && fwrite(h, 1, bytes, f) != bytes) die("write", "output file");
  free(h);
}

int main(int argc, char** argv) {
  if (argc != 3) die("usage", "abi_step IN OUT");
  if (dspark_abi_version() != DSPARK_ABI_VERSION) die("libdspark", "ABI version mismatch");
  FILE* in = fopen(argv[1], "rb");
  if (!in) die("open", argv[1]);
  int32_t dims[4];
  int64_t K;
  if (fread(dims, sizeof(int32_t), 4, in) != 4 || fread(&K, sizeof(int64_t), 1, in) != 1) die("read", "header");
  const int32_t R = dims[0], gamma = dims[1], V = dims[2], rank = dims[3];
  if (R < 1 || gamma < 1 || V < 1 || rank < 1) die("read", "bad sizes");
  const size_t RG = (size_t)R * gamma;

  /* inputs: the target rows stay on the host until the schedule is known */
  float* U = (float*)dev_read(in, RG * V * sizeof(float));
  float* target_h = (float*)malloc((size_t)R * (gamma + 1) * V * sizeof(float));
  if (!target_h) die("malloc", "out of memory");
  if (fread(target_h, sizeof(float), (size_t)R * (gamma + 1) * V, in) != (size_t)R * (gamma + 1) * V)
    die("read", "target");
  void* W1 = dev_read(in, (size_t)V * rank * 2);
  void* W2 = dev_read(in, (size_t)V * rank * 2);
  int32_t* anchor = (int32_t*)dev_read(in, R * sizeof(int32_t));
  float* temp = (float*)dev_read(in, R * sizeof(float));
  float* u_draft = (float*)dev_read(in, RG * sizeof(float));
  float* u_accept = (float*)dev_read(in, RG * sizeof(float));
  float* u_final = (float*)dev_read(in, R * sizeof(float));
  float* c = (float*)dev_read(in, RG * sizeof(float));
  fclose(in);

  /* draft */
  int32_t* y = (int32_t*)dev_alloc(RG * sizeof(int32_t));
  float* q_tok = (float*)dev_alloc(RG * sizeof(float));
  float* q_stats = (float*)dev_alloc(RG * 2 * sizeof(float));
  dspark_draft_args da;
  memset(&da, 0, sizeof(da));
  da.struct_size = sizeof(da);
  da.R = R;
  da.gamma = gamma;
  da.V = V;
  da.rank = rank;
  da.wdtype = DSPARK_W_BF16;
  da.head = DSPARK_HEAD_MARKOV;
  size_t ws_bytes = 0;
  ds_ok(dspark_draft_workspace_size(&da, &ws_bytes), "dspark_draft_workspace_size");
  da.U = U;
  da.W1 = W1;
  da.W2 = W2;
  da.anchor = anchor;
  da.temp = temp;
  da.u_draft = u_draft;
  da.y = y;
  da.q_tok = q_tok;
  da.q_stats = q_stats;
  da.workspace = dev_alloc(ws_bytes);
  da.workspace_bytes = ws_bytes;
  da.stream = NULL;
  ds_ok(dspark_draft_block(&da), "dspark_draft_block");

  /* schedule */
  const int64_t n_rows_max = dspark_schedule_rows(R, gamma, K);
  if (n_rows_max < R) die("dspark_schedule_rows", "bad row count");
  dspark_schedule_args sa;
  memset(&sa, 0, sizeof(sa));
  sa.struct_size = sizeof(sa);
  sa.R = R;
  sa.gamma = gamma;
  sa.K = K;
  sa.c = c;
  sa.anchor = anchor;
  sa.y = y;
  sa.a = (float*)dev_alloc(RG * sizeof(float));
  sa.l = (int32_t*)dev_alloc(R * sizeof(int32_t));
  sa.row_offsets = (int32_t*)dev_alloc((R + 1) * sizeof(int32_t));
  sa.row_req = (int32_t*)dev_alloc(n_rows_max * sizeof(int32_t));
  sa.row_pos = (int32_t*)dev_alloc(n_rows_max * sizeof(int32_t));
  sa.row_tok = (int32_t*)dev_alloc(n_rows_max * sizeof(int32_t));
  size_t sws = 0;
  ds_ok(dspark_schedule_workspace_size(&sa, &sws), "dspark_schedule_workspace_size");
  if (sws != 0) die("dspark_schedule_workspace_size", "a schedule without checks needs no workspace");
  ds_ok(dspark_schedule(&sa), "dspark_schedule");
  hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");

  /* the target rows of the schedule, gathered on the host */
  int32_t* off_h = (int32_t*)malloc((R + 1) * sizeof(int32_t));
  if (!off_h) die("malloc", "out of memory");
  hip_ok(hipMemcpy(off_h, sa.row_offsets, (R + 1) * sizeof(int32_t), hipMemcpyDeviceToHost), "offsets");
  const int64_t n_rows = off_h[R];
  if (n_rows < R || n_rows > n_rows_max) die("dspark_schedule", "row count out of range");
  int32_t* req_h = (int32_t*)malloc(n_rows * sizeof(int32_t));
  int32_t* pos_h = (int32_t*)malloc(n_rows * sizeof(int32_t));
  float* rows_h = (float*)malloc((size_t)n_rows * V * sizeof(float));
  if (!req_h || !pos_h || !rows_h) die("malloc", "out of memory");
  hip_ok(hipMemcpy(req_h, sa.row_req, n_rows * sizeof(int32_t), hipMemcpyDeviceToHost), "row_req");
  hip_ok(hipMemcpy(pos_h, sa.row_pos, n_rows * sizeof(int32_t), hipMemcpyDeviceToHost), "row_pos");
  for (int64_t i = 0; i < n_rows; ++i) {
    if (req_h[i] < 0 || req_h[i] >= R || pos_h[i] < 0 || pos_h[i] > gamma) die("dspark_schedule", "bad row");
    memcpy(rows_h + (size_t)i * V, target_h + ((size_t)req_h[i] * (gamma + 1) + pos_h[i]) * V, V * sizeof(float));
  }
  float* rows = (float*)dev_alloc((size_t)n_rows * V * sizeof(float));
  hip_ok(hipMemcpy(rows, rows_h, (size_t)n_rows * V * sizeof(float), hipMemcpyHostToDevice), "rows");

  /* verify */
  int32_t* n_accept = (int32_t*)dev_alloc(R * sizeof(int32_t));
  int32_t* out_tok = (int32_t*)dev_alloc(R * sizeof(int32_t));
  float* p_tok = (float*)dev_alloc(RG * sizeof(float));
  dspark_verify_args va;
  memset(&va, 0, sizeof(va));
  va.struct_size = sizeof(va);
  va.R = R;
  va.gamma = gamma;
  va.V = V;
  va.rank = rank;
  va.wdtype = DSPARK_W_BF16;
  va.head = DSPARK_HEAD_MARKOV;
  va.n_rows = n_rows;
  size_t vws = 0;
  ds_ok(dspark_verify_workspace_size(&va, &vws), "dspark_verify_workspace_size");
  va.target = rows;
  va.row_offsets = sa.row_offsets;
  va.U = U;
  va.W1 = W1;
  va.W2 = W2;
  va.anchor = anchor;
  va.temp = temp;
  va.y = y;
  va.q_tok = q_tok;
  va.q_stats = q_stats;
  va.u_accept = u_accept;
  va.u_final = u_final;
  va.n_accept = n_accept;
  va.out_tok = out_tok;
  va.p_tok = p_tok;
  va.workspace = dev_alloc(vws);
  va.workspace_bytes = vws;
  va.stream = NULL;
  ds_ok(dspark_verify(&va), "dspark_verify");
  hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");

  FILE* out = fopen(argv[2], "wb");
  if (!out) die("open", argv[2]);
  host_write(out, y, RG * sizeof(int32_t));
  host_write(out, q_tok, RG * sizeof(float));
  host_write(out, q_stats, RG * 2 * sizeof(float));
  host_write(out, sa.l, R * sizeof(int32_t));
  host_write(out, sa.row_offsets, (R + 1) * sizeof(int32_t));
  host_write(out, n_accept, R * sizeof(int32_t));
  host_write(out, out_tok, R * sizeof(int32_t));
  host_write(out, p_tok, RG * sizeof(float));
  if (fclose(out) != 0) die("close", argv[2]);
  return 0;
}
