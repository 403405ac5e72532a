"""MI355X-native Llama-2 decoder layer (prefill + KV-cached decode).

The compute path is the C-ABI library ``libllama_layer.so`` built from
``csrc/``; ``binding`` marshals torch tensors into it.  Importing the package
loads nothing: the library is opened on first use.
"""
