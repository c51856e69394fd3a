// ABI-level helpers of libpuro: status strings and version.
#include "common.hpp"

extern "C" const char* puro_status_string(int status) {
  switch (status) {
    case PURO_OK: return "PURO_OK";
    case PURO_ERR_NULL: return "PURO_ERR_NULL: required pointer is NULL";
    case PURO_ERR_SHAPE: return "PURO_ERR_SHAPE: dimension negative, not a multiple of 128, or too large";
    case PURO_ERR_ALIGN: return "PURO_ERR_ALIGN: tensor pointer not 16-byte aligned";
    case PURO_ERR_LAUNCH: return "PURO_ERR_LAUNCH: kernel launch failed";
    case PURO_ERR_ARG: return "PURO_ERR_ARG: argument out of range";
    case PURO_ERR_INPUT: return "PURO_ERR_INPUT: input data outside the contract (debug check)";
    default: return "unknown puro_status";
  }
}

extern "C" int puro_abi_version(void) { return 1; }
