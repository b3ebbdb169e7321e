/*
 * A plain C caller of the library (test infrastructure): it includes only
 * bqd.h and the HIP runtime API, reads raw inputs from a directory, runs
 * cq_prepare_matvec, cq_gather_rows, f8_matvec, logits_sample,
 * f8_matvec_argmax and f8_matvec_sample on a stream of its own, and writes the outputs back to the
 * directory for the test to compare with the oracle.
 *
 * usage: caller DIR
 * DIR/shape.txt: "R C Cp G BITS ROW_BYTES N_IDS FR FC SR SC NL K" (CQ matrix,
 * gather ids, F8 matrix and scale grid, logits, top-k); raw little-endian inputs
 * packed.bin (uint8 R x ROW_BYTES), norms.bin (uint16 R x Cp/G), codebook.bin
 * (float 2^BITS), x.bin (float C), ids.bin (int32 N_IDS), f8_w.bin (uint8
 * FR x FC), f8_s.bin (uint8 SR x SC), f8_x.bin (float FC), logits.bin (float NL),
 * state.bin (uint32).
 * Outputs: prepared.bin, y.bin, gathered.bin, f8_y.bin, token.bin, topk_ids.bin,
 * topk_logits.bin, state_out.bin, argmax_y.bin, argmax_token.bin, sample_y.bin,
 * sample_token.bin, sample_ids.bin, sample_logits.bin, sample_state_out.bin
 * (f8_matvec_sample: top K of the F8 matvec's outputs, drawn at temperature
 * 0.8 from its own copy of the initial state).
 */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "bqd.h"

static const char *dir;

static void fail(const char *what, const char *why)
{
    fprintf(stderr, "caller: %s: %s\n", what, why);
    exit(1);
}

#define HIP_OK(call)                                                  \
    do {                                                              \
        hipError_t e_ = (call);                                       \
        if (e_ != hipSuccess) fail(#call, hipGetErrorString(e_));     \
    } while (0)

#define BQD_OK_(call)                                                 \
    do {                                                              \
        int s_ = (call);                                              \
        if (s_ != BQD_OK) fail(#call, bqd_status_string(s_));         \
    } while (0)

static FILE *open_in_dir(const char *name, const char *mode)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, mode);
    if (!f) fail(path, "cannot open");
    return f;
}

/* `bytes` bytes of DIR/name into a new device buffer. */
static void *load_to_device(const char *name, size_t bytes)
{
    void *h = malloc(bytes ? bytes : 1), *d = NULL;
    if (!h) fail(name, "out of host memory");
    FILE *f = open_in_dir(name, "rb");
    if (fread(h, 1, bytes, f) != bytes) fail(name, "short file");
    fclose(f);
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    free(h);
    return d;
}

static void *device_zeros(size_t bytes)
{
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    HIP_OK(hipMemset(d, 0, bytes ? bytes : 1));
    return d;
}

static void save_from_device(const char *name, const void *d, size_t bytes)
{
    void *h = malloc(bytes ? bytes : 1);
    if (!h) fail(name, "out of host memory");
    HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    FILE *f = open_in_dir(name, "wb");
    if (fwrite(h, 1, bytes, f) != bytes) fail(name, "short write");
    fclose(f);
    free(h);
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 2;
    }
    dir = argv[1];
    long long R, C, Cp, G, B, RB, NI, FR, FC, SR, SC, NL, K;
    FILE *f = open_in_dir("shape.txt", "r");
    if (fscanf(f, "%lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld", &R, &C, &Cp,
               &G, &B, &RB, &NI, &FR, &FC, &SR, &SC, &NL, &K) != 13)
        fail("shape.txt", "expected 13 integers");
    fclose(f);

    bqd_cq_matrix m;
    m.output = R;
    m.input = C;
    m.input_padded = Cp;
    m.group = G;
    m.bits = B;
    m.row_bytes = RB;
    m.packed = load_to_device("packed.bin", (size_t)(R * RB));
    m.norms = load_to_device("norms.bin", (size_t)(R * (Cp / G)) * 2);
    m.codebook = load_to_device("codebook.bin", (size_t)4 << B);
    const float *x = load_to_device("x.bin", (size_t)C * 4);
    const int32_t *ids = load_to_device("ids.bin", (size_t)NI * 4);
    const uint8_t *fw = load_to_device("f8_w.bin", (size_t)(FR * FC));
    const uint8_t *fs = load_to_device("f8_s.bin", (size_t)(SR * SC));
    const float *fx = load_to_device("f8_x.bin", (size_t)FC * 4);
    const float *logits = load_to_device("logits.bin", (size_t)NL * 4);
    uint32_t *state = load_to_device("state.bin", 4);
    uint32_t *sstate = load_to_device("state.bin", 4);

    float *prepared = device_zeros((size_t)Cp * 4);
    float *y = device_zeros((size_t)R * 4);
    float *gathered = device_zeros((size_t)(NI * C) * 4);
    float *fy = device_zeros((size_t)FR * 4);
    int32_t *token = device_zeros(4);
    int32_t *topk_ids = device_zeros((size_t)K * 4);
    float *topk_logits = device_zeros((size_t)K * 4);
    const int64_t ws_bytes = logits_sample_workspace_bytes(NL, K);
    if (ws_bytes < 0) fail("logits_sample_workspace_bytes", bqd_status_string((int)ws_bytes));
    void *ws = device_zeros((size_t)ws_bytes);
    float *ay = device_zeros((size_t)FR * 4);
    int32_t *atok = device_zeros(4);
    const int64_t aws_bytes = f8_matvec_argmax_workspace_bytes(1);
    if (aws_bytes < 0)
        fail("f8_matvec_argmax_workspace_bytes", bqd_status_string((int)aws_bytes));
    void *aws = device_zeros((size_t)aws_bytes);
    float *sy = device_zeros((size_t)FR * 4);
    int32_t *stok = device_zeros(4);
    int32_t *sids = device_zeros((size_t)K * 4);
    float *svals = device_zeros((size_t)K * 4);
    void *sws = device_zeros((size_t)aws_bytes);

    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    BQD_OK_(cq_prepare_matvec(&m, x, prepared, y, 1, 0, R, s));
    BQD_OK_(cq_gather_rows(&m, ids, NI, gathered, s));
    BQD_OK_(f8_matvec(fw, FR, FC, fs, SR, SC, fx, fy, 1, s));
    /* top K of the logits and one draw at temperature 0.8 */
    BQD_OK_(logits_sample(logits, NL, K, 0.8f, state, ws, ws_bytes, token, topk_ids, topk_logits,
                          s));
    BQD_OK_(f8_matvec_argmax(fw, FR, FC, fs, SR, SC, fx, ay, 1, aws, aws_bytes, atok, s));
    BQD_OK_(f8_matvec_sample(fw, FR, FC, fs, SR, SC, fx, sy, 1, K, 0.8f, sstate, sws, aws_bytes,
                             stok, sids, svals, s));
    HIP_OK(hipStreamSynchronize(s));

    save_from_device("prepared.bin", prepared, (size_t)Cp * 4);
    save_from_device("y.bin", y, (size_t)R * 4);
    save_from_device("gathered.bin", gathered, (size_t)(NI * C) * 4);
    save_from_device("f8_y.bin", fy, (size_t)FR * 4);
    save_from_device("token.bin", token, 4);
    save_from_device("topk_ids.bin", topk_ids, (size_t)K * 4);
    save_from_device("topk_logits.bin", topk_logits, (size_t)K * 4);
    save_from_device("state_out.bin", state, 4);
    save_from_device("argmax_y.bin", ay, (size_t)FR * 4);
    save_from_device("argmax_token.bin", atok, 4);
    save_from_device("sample_y.bin", sy, (size_t)FR * 4);
    save_from_device("sample_token.bin", stok, 4);
    save_from_device("sample_ids.bin", sids, (size_t)K * 4);
    save_from_device("sample_logits.bin", svals, (size_t)K * 4);
    save_from_device("sample_state_out.bin", sstate, 4);
    HIP_OK(hipStreamDestroy(s));
    printf("caller: ok\n");
    return 0;
}
