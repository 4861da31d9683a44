/*
 * A plain C99 client of include/mccb.h, built and run by tests/test_c_client.py on the CPU: the
 * header must compile as C without HIP headers, and the library's host-only entry points (phase 1,
 * the plan, status strings, validation that rejects arguments before any HIP call) must behave
 * the same when called from C as through the Python binding. It prints one "name value" line per
 * check.
 */
#include <stdint.h>
#include <stdio.h>

#include "mccb.h"

int main(void) {
    uint64_t ws = 0;
    int rc = mccb_get_workspace_size(16384, 32, 5120, MCCB_BF16, &ws);
    printf("ws_rc %d\nws_bytes %llu\n", rc, (unsigned long long)ws);

    mccb_plan_t plan;
    rc = mccb_get_plan(16384, 32, 5120, MCCB_BF16, &plan);
    printf("plan_rc %d\n", rc);
    printf("rows_per_strip %lld\nn_strips %lld\nplan_ws %llu\n", (long long)plan.rows_per_strip,
           (long long)plan.n_strips, (unsigned long long)plan.workspace_size);

    printf("null_out %d\n", mccb_get_workspace_size(64, 1, 384, MCCB_BF16, NULL));
    printf("bad_dtype %d\n", mccb_get_workspace_size(64, 1, 384, 7, &ws));
    printf("bad_H %d\n", mccb_get_workspace_size(64, 1, 100, MCCB_FP16, &ws));
    printf("bad_BS %d\n", mccb_get_workspace_size(524289, 1, 384, MCCB_FP16, &ws));

    /* phase 2 with a NULL input: rejected on the host, nothing enqueued, no HIP call */
    rc = mccb_backward(NULL, NULL, NULL, NULL, NULL, NULL, 64, 1, 384, MCCB_BF16, NULL, 0, NULL);
    printf("backward_null %d\n", rc);
    rc = mccb_forward(NULL, NULL, NULL, NULL, 64, 1, 384, MCCB_BF16, NULL);
    printf("forward_null %d\n", rc);

    printf("str_ok %s\n", mccb_status_string(MCCB_OK));
    printf("str_shape %s\n", mccb_status_string(MCCB_ERR_SHAPE));
    printf("str_unknown %s\n", mccb_status_string(12345));
    return 0;
}
