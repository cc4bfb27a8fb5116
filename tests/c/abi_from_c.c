/* Calls libqknorm.so from plain C through include/qknorm.h, with no GPU work:
 * the ABI version, a plan description for the GQA prefill shape, and an
 * argument error with its message. Built and run by tests/test_c_abi.py. */
#include <stdio.h>
#include <string.h>

#include "qknorm.h"

int main(void) {
  if (qknorm_abi_version() != 3) {
    printf("abi version %d\n", qknorm_abi_version());
    return 1;
  }
  /* stand-in device addresses: never dereferenced by planning */
  const uintptr_t base = (uintptr_t)1 << 32, out = (uintptr_t)1 << 44, gam = (uintptr_t)1 << 46;
  qknorm_operand_t q = {(const void*)base, 7168, (void*)(base + out), 7168, (const void*)gam, 5120};
  qknorm_operand_t k = {(const void*)(base + 5120 * 2), 7168, (void*)(base + out + 5120 * 2), 7168,
                        (const void*)(gam + 65536), 1024};
  char buf[512];
  int rc = qknorm_describe_plan(QKNORM_OP_FUSED, &q, &k, 8192, QKNORM_BF16, 1, buf, sizeof buf);
  if (rc != QKNORM_OK || strstr(buf, "slots=3") == NULL) {
    printf("describe_plan rc=%d '%s'\n", rc, buf);
    return 1;
  }
  printf("plan: %s\n", buf);
  /* shards that do not divide the widths: rejected before any launch */
  rc = qknorm_fused(&q, &k, 8192, QKNORM_BF16, 1e-6f, 3, NULL);
  if (rc != QKNORM_ERR_INVALID_ARG || strncmp(qknorm_last_error(), "qknorm_fused:", 13) != 0) {
    printf("fused rc=%d '%s'\n", rc, qknorm_last_error());
    return 1;
  }
  printf("error: %s\n", qknorm_last_error());
  return 0;
}
