/*
 * pkv_status.h -- status codes shared by every entry point of the paged
 * KV-cache library (pkv.h, pkv_alloc.h).  0 is success, errors are negative.
 */
#ifndef PKV_STATUS_H_
#define PKV_STATUS_H_

enum {
  PKV_OK = 0,
  PKV_E_NULL = -1,         /* a required pointer is NULL                       */
  PKV_E_SHAPE = -2,        /* sizes inconsistent, out of range or misaligned   */
  PKV_E_UNSUPPORTED = -3,  /* dtype / head_dim / block_size / group not built  */
  PKV_E_WORKSPACE = -4,    /* workspace missing or smaller than required       */
  PKV_E_HIP = -5,          /* a kernel launch failed                           */
  PKV_E_NOMEM = -6,        /* allocator: not enough free blocks                */
  PKV_E_NOSEQ = -7,        /* allocator: unknown sequence id                   */
  PKV_E_EXISTS = -8        /* allocator: sequence id already present           */
};

#endif /* PKV_STATUS_H_ */
