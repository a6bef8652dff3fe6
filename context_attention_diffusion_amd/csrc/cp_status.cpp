// Version and status strings of the libcpattn C ABI.
#include "cp_attn.h"

extern "C" int cp_abi_version(void) { return CP_ABI_VERSION; }

extern "C" const char* cp_status_string(int status) {
  switch (status) {
    case CP_OK: return "ok";
    case CP_ERR_NULL: return "a required pointer is NULL";
    case CP_ERR_DTYPE: return "dtype not supported by this entry point";
    case CP_ERR_SHAPE: return "invalid or too large shape (sizes must be >= 1 and within the supported extent)";
    case CP_ERR_DIVISIBILITY: return "shape not divisible (heads must divide by W; chunks must split evenly)";
    case CP_ERR_HEAD_DIM: return "head dim not supported (layout: multiple of 8; attention: 64 or 128)";
    case CP_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case CP_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case CP_ERR_SCALE: return "softmax scale must be finite and > 0";
    case CP_ERR_UNSUPPORTED: return "unsupported request (unknown phase or layout flag, or too many ranks)";
    case CP_ERR_HIP: return "HIP runtime error while enqueueing the kernel";
    case CP_ERR_WORKSPACE: return "attention workspace too small (see cp_attn_workspace_bytes)";
    case CP_ERR_SCRATCH: return "problem needs more than the library's static scratch array (CP_ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status code";
  }
}
