/* Plain C consumer of libqlinear.so: exercises the host-side validation of
 * the C ABI (every call here is rejected before any HIP call, so no GPU is
 * needed) and prints one line per check.  Built and run by test_abi_c.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qlinear.h"

static int failures = 0;

static void expect(const char *what, qlin_status got, qlin_status want)
{
    printf("%-44s %d %s\n", what, (int)got, got == want ? "ok" : "FAIL");
    if (got != want)
        ++failures;
}

int main(void)
{
    /* fake, aligned device addresses: never dereferenced on these paths */
    const void *A = (const void *)0x10000, *B = (const void *)0x20000;
    void *Y = (void *)0x30000;
    const float *s = (const float *)0x40000;
    float *so = (float *)0x40000;
    qlin_config c;

    expect("abi version", qlin_abi_version() == QLINEAR_ABI_VERSION ? QLIN_OK : QLIN_ERR_HIP, QLIN_OK);
    expect("K not a multiple of 16",
           qlin_scaled_mm(QLIN_INT8, 4, 64, 40, A, 48, s, B, 48, s, Y, 64, NULL, 0, NULL),
           QLIN_ERR_BAD_SHAPE);
    expect("negative M",
           qlin_scaled_mm(QLIN_E4M3, -1, 64, 64, A, 64, s, B, 64, s, Y, 64, NULL, 0, NULL),
           QLIN_ERR_BAD_SHAPE);
    expect("empty M is a no-op",
           qlin_scaled_mm(QLIN_E4M3, 0, 64, 64, NULL, 64, NULL, NULL, 64, NULL, NULL, 64, NULL, 0, NULL),
           QLIN_OK);
    expect("null A",
           qlin_scaled_mm(QLIN_E4M3, 4, 64, 64, NULL, 64, s, B, 64, s, Y, 64, NULL, 0, NULL),
           QLIN_ERR_NULL_POINTER);
    expect("lda < K",
           qlin_scaled_mm(QLIN_E4M3, 4, 64, 128, A, 64, s, B, 128, s, Y, 64, NULL, 0, NULL),
           QLIN_ERR_BAD_STRIDE);
    expect("misaligned B",
           qlin_scaled_mm(QLIN_E4M3, 4, 64, 64, A, 64, s, (const char *)B + 4, 64, s, Y, 64, NULL, 0, NULL),
           QLIN_ERR_MISALIGNED);
    expect("block: N not a multiple of 128",
           qlin_block_scaled_mm(4, 100, 256, A, 256, s, B, 256, s, Y, 100, NULL, 0, NULL),
           QLIN_ERR_BAD_SHAPE);
    expect("bad dtype",
           qlin_scaled_mm((qlin_dtype)5, 4, 64, 64, A, 64, s, B, 64, s, Y, 64, NULL, 0, NULL),
           QLIN_ERR_BAD_ARGUMENT);
    expect("select config", qlin_select_config(QLIN_TOKEN_CHANNEL, QLIN_INT8, 16, 4096, 2048, &c), QLIN_OK);
    c.split_k = 3;
    expect("split_k not a power of two",
           qlin_check_config(QLIN_TOKEN_CHANNEL, QLIN_INT8, 16, 4096, 2048, &c), QLIN_ERR_BAD_CONFIG);
    c.split_k = 4;
    c.reduce = QLIN_REDUCE_LAST_ARRIVER;
    expect("split config accepted", qlin_check_config(QLIN_TOKEN_CHANNEL, QLIN_INT8, 16, 4096, 2048, &c),
           QLIN_OK);
    expect("workspace required",
           qlin_scaled_mm_cfg(QLIN_INT8, 16, 4096, 2048, A, 2048, s, B, 2048, s, Y, 4096, NULL, 0, NULL, &c),
           QLIN_ERR_WORKSPACE);
    expect("workspace size > 0",
           qlin_workspace_size(QLIN_TOKEN_CHANNEL, QLIN_INT8, 16, 4096, 2048, &c) > 0 ? QLIN_OK : QLIN_ERR_WORKSPACE,
           QLIN_OK);
    expect("fused rms norm: K % 16",
           qlin_rms_norm_dynamic_per_token_quant(QLIN_E4M3, 4, 40, A, 48, NULL, 0, B, 1e-6f, Y, 48, so, NULL),
           QLIN_ERR_BAD_SHAPE);
    expect("fused rms norm per block: K % 128",
           qlin_rms_norm_per_block_quant(4, 144, A, 144, NULL, 0, B, 1e-6f, Y, 144, so, NULL),
           QLIN_ERR_BAD_SHAPE);
    expect("fused silu: rows of 2K",
           qlin_silu_and_mul_dynamic_per_token_quant(QLIN_INT8, 4, 64, A, 64, Y, 64, so, NULL),
           QLIN_ERR_BAD_STRIDE);
    expect("fused silu per block: empty",
           qlin_silu_and_mul_per_block_quant(0, 128, NULL, 256, NULL, 128, NULL, NULL), QLIN_OK);
    expect("missing table file", qlin_load_config_table("/nonexistent/qlin.cfg"), QLIN_ERR_CONFIG_FILE);
    expect("restore compiled-in table", qlin_load_config_table(NULL), QLIN_OK);
    qlin_config k0;
    int32_t mask = 0;
    expect("kernel instance 0", qlin_kernel_instance(0, &k0, &mask), QLIN_OK);
    expect("status string", strlen(qlin_status_string(QLIN_ERR_HIP)) > 0 ? QLIN_OK : QLIN_ERR_HIP, QLIN_OK);
    printf("%s\n", failures ? "FAILED" : "ALL OK");
    return failures ? 1 : 0;
}
